"""Thin ctypes binding over libtokengate.so (include/tokengate.h).

Functions carry the C names.  They take torch tensors that live on the GPU,
marshal their data pointers, sizes and torch's current HIP stream, and call
the C ABI; every step of the computation runs in the library's HIP kernels.
PyTorch is used only to own device memory and to provide the stream.  Output
tensors may be passed in (no allocation) or are allocated here with
``torch.empty`` on the input's device.  A missing library raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtokengate.so")

TG_OK, TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_HIP = 0, 1, 2, 3, 4
TG_FP32, TG_BF16 = 0, 1

_c_vp = ctypes.c_void_p
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_f32 = ctypes.c_float
_c_f64 = ctypes.c_double

# name -> (argtypes, restype)
SIGNATURES = {
    "tg_abi_version": ([], ctypes.c_int),
    "tg_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "tg_last_error": ([], ctypes.c_char_p),
    "tg_gate_score": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_f32,
                       _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_gate_select": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_f32, _c_i64,
                        _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp], ctypes.c_int),
    "tg_gate_select_gather": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_f32,
                               _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp],
                              ctypes.c_int),
    "tg_select_topk": ([_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp], ctypes.c_int),
    "tg_select_topk_workspace_size": ([_c_i64], _c_i64),
    "tg_select_topk_ws": ([_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp], ctypes.c_int),
    "tg_select_topk_varlen": ([_c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
                              ctypes.c_int),
    "tg_gather": ([ctypes.c_int, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp,
                   _c_vp], ctypes.c_int),
    "tg_gather_varlen": ([ctypes.c_int, _c_vp, _c_vp, _c_i32, _c_i64, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp,
                          _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_rope_table": ([_c_vp, _c_i64, _c_i32, _c_f64, _c_vp], ctypes.c_int),
    "tg_rope_kv": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp,
                    _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_gated_attn": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                       _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_gated_attn_varlen": ([ctypes.c_int, _c_vp, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_f32,
                              _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_gated_attn_ex": ([ctypes.c_int, _c_vp, _c_i32, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_f32, _c_vp,
                          _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_linear": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64,
                   _c_vp], ctypes.c_int),
    "tg_swiglu": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp],
                  ctypes.c_int),
    "tg_qkv_proj": ([ctypes.c_int, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp,
                     _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_check_positions": ([_c_vp, _c_i64, _c_vp, _c_i32, _c_vp, _c_vp], ctypes.c_int),
    "tg_decode_attn_workspace_size": ([_c_i32, _c_i64, _c_i32, _c_i32, _c_i32], _c_i64),
    "tg_decode_attn_noalloc_max_bytes": ([], _c_i64),
    "tg_decode_attn_noalloc": ([ctypes.c_int, _c_vp, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_f32, _c_vp, _c_vp,
                                _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "tg_decode_attn": ([ctypes.c_int, _c_vp, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp,
                        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp], ctypes.c_int),
}

_LIB: Optional[ctypes.CDLL] = None


class TokenGateError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str):
        super().__init__(f"{func}: {status_string(status)}: {detail}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libtokengate.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"libtokengate.so not found at {path}; build it with "
                           "`python -m learned_token_pruning_03_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tg_status_string(status).decode()


def _check(func: str, status: int) -> None:
    if status != TG_OK:
        raise TokenGateError(func, status, load_library().tg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of t for the C ABI (which takes device pointers only)."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> Optional[int]:
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TG_BF16
    if t.dtype == torch.float32:
        return TG_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# The C ABI takes raw pointers and no buffer lengths, so these checks are the
# only guard against a call that would read or write past a tensor.
def _vec(t: Optional[torch.Tensor], n: int, dtype: torch.dtype, name: str) -> None:
    """t is None, or a contiguous GPU tensor of `dtype` with at least n elements."""
    if t is None:
        return
    _need(t.dtype == dtype and t.is_contiguous() and t.numel() >= n,
          f"{name} must be a contiguous {dtype} tensor with at least {n} elements")
    _need(t.device.type == "cuda", f"{name} must live on the GPU")


def _like(t: torch.Tensor, shape, dtype: torch.dtype, name: str) -> None:
    """t is a contiguous GPU tensor of exactly `shape` and `dtype`."""
    _need(tuple(t.shape) == tuple(shape) and t.dtype == dtype and t.is_contiguous(),
          f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    _need(t.device.type == "cuda", f"{name} must live on the GPU")


# ---------------------------------------------------------------------------
def tg_gate_score(h: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                  b2: float, g: Optional[torch.Tensor] = None, s: Optional[torch.Tensor] = None,
                  want_scores: bool = False):
    """g [n] fp32 (and s [n] if requested) for h [n, d], W1 [hidden, d]."""
    lib = load_library()
    _need(h.dim() == 2 and h.stride(1) == 1, "h must be [n, d] with unit column stride")
    n, d = h.shape
    hidden = w1.shape[0]
    _need(w1.shape == (hidden, d) and w1.is_contiguous() and w1.dtype == h.dtype, "w1 must be [hidden, d]")
    _need(w2.numel() == hidden and w2.dtype == torch.float32, "w2 must be fp32 [hidden]")
    _need(b1 is None or (b1.numel() == hidden and b1.dtype == torch.float32), "b1 must be fp32 [hidden]")
    if g is None:
        g = torch.empty(n, dtype=torch.float32, device=h.device)
    if want_scores and s is None:
        s = torch.empty(n, dtype=torch.float32, device=h.device)
    _check("tg_gate_score", lib.tg_gate_score(_dtype_code(h), n, d, hidden, _ptr(h), h.stride(0), _ptr(w1),
                                              _ptr(b1), _ptr(w2), float(b2), _ptr(g), _ptr(s), _stream(h)))
    return (g, s) if want_scores or s is not None else g


def select_workspace(n: int, device) -> torch.Tensor:
    """A zero-filled select workspace for prompts of up to n tokens, as
    tg_gate_select needs on first use (every call leaves it zero-filled)."""
    return torch.zeros(max(tg_select_topk_workspace_size(n), 16), dtype=torch.uint8, device=device)


def _check_gate_inputs(h, w1, b1, w2):
    _need(h.dim() == 2 and h.stride(1) == 1, "h must be [n, d] with unit column stride")
    n, d = h.shape
    hidden = w1.shape[0]
    _need(w1.shape == (hidden, d) and w1.is_contiguous() and w1.dtype == h.dtype, "w1 must be [hidden, d]")
    _need(w2.numel() == hidden and w2.dtype == torch.float32 and w2.is_contiguous(), "w2 must be fp32 [hidden]")
    _need(b1 is None or (b1.numel() == hidden and b1.dtype == torch.float32 and b1.is_contiguous()),
          "b1 must be fp32 [hidden]")
    return n, d, hidden


def tg_gate_select(h: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor, b2: float,
                   k: int, q_len: int, g: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, s: Optional[torch.Tensor] = None,
                   want_scores: bool = False):
    """Gate scores and the top-K selection over them in one call; returns
    (g, idx), or (g, s, idx) when scores are requested.  `workspace` must be
    a zero-filled uint8 tensor the first time it is used (select_workspace)."""
    lib = load_library()
    n, d, hidden = _check_gate_inputs(h, w1, b1, w2)
    kept = min(int(k), n)
    g = torch.empty(n, dtype=torch.float32, device=h.device) if g is None else g
    idx = torch.empty(kept, dtype=torch.int32, device=h.device) if idx is None else idx
    if want_scores and s is None:
        s = torch.empty(n, dtype=torch.float32, device=h.device)
    _vec(g, n, torch.float32, "g")
    _vec(s, n, torch.float32, "s")
    _vec(idx, kept, torch.int32, "idx")
    if workspace is None:
        workspace = select_workspace(n, h.device)
    _need(workspace.is_contiguous() and workspace.device == h.device, "workspace must be a contiguous device tensor")
    _check("tg_gate_select",
           lib.tg_gate_select(_dtype_code(h), n, d, hidden, _ptr(h), h.stride(0), _ptr(w1), _ptr(b1), _ptr(w2),
                              float(b2), int(k), int(q_len), _ptr(g), _ptr(s), _ptr(idx), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(h)))
    return (g, s, idx) if (want_scores or s is not None) else (g, idx)


def tg_gate_select_gather(h: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                          b2: float, k: int, q_len: int, g: Optional[torch.Tensor] = None,
                          idx: Optional[torch.Tensor] = None, h_out: Optional[torch.Tensor] = None,
                          g_out: Optional[torch.Tensor] = None, pos_out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """Gate, top-K select and gather of the kept rows in two kernels; returns
    (g, idx, h_out, g_out, pos_out).  Workspace as tg_gate_select."""
    lib = load_library()
    n, d, hidden = _check_gate_inputs(h, w1, b1, w2)
    kept = min(int(k), n)
    dev = h.device
    g = torch.empty(n, dtype=torch.float32, device=dev) if g is None else g
    idx = torch.empty(kept, dtype=torch.int32, device=dev) if idx is None else idx
    h_out = torch.empty(kept, d, dtype=h.dtype, device=dev) if h_out is None else h_out
    g_out = torch.empty(kept, dtype=torch.float32, device=dev) if g_out is None else g_out
    pos_out = torch.empty(kept, dtype=torch.int32, device=dev) if pos_out is None else pos_out
    _vec(g, n, torch.float32, "g")
    _vec(idx, kept, torch.int32, "idx")
    _like(h_out, (kept, d), h.dtype, "h_out")
    _vec(g_out, kept, torch.float32, "g_out")
    _vec(pos_out, kept, torch.int32, "pos_out")
    if workspace is None:
        workspace = select_workspace(n, dev)
    _need(workspace.is_contiguous() and workspace.device == dev, "workspace must be a contiguous device tensor")
    _check("tg_gate_select_gather",
           lib.tg_gate_select_gather(_dtype_code(h), n, d, hidden, _ptr(h), h.stride(0), _ptr(w1), _ptr(b1),
                                     _ptr(w2), float(b2), int(k), int(q_len), _ptr(g), None, _ptr(idx), _ptr(h_out),
                                     _ptr(g_out), _ptr(pos_out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(h)))
    return g, idx, h_out, g_out, pos_out


def tg_select_topk(g: torch.Tensor, k: int, q_len: int, idx: Optional[torch.Tensor] = None):
    """Ascending int32 indices of the min(k, n) kept tokens."""
    lib = load_library()
    _need(g.dim() == 1 and g.dtype == torch.float32 and g.is_contiguous(), "g must be contiguous fp32 [n]")
    n = g.shape[0]
    kept = min(int(k), n)
    if idx is None:
        idx = torch.empty(kept, dtype=torch.int32, device=g.device)
    _vec(idx, kept, torch.int32, "idx")
    _check("tg_select_topk", lib.tg_select_topk(_ptr(g), n, int(k), int(q_len), _ptr(idx), _stream(g)))
    return idx


def tg_select_topk_workspace_size(n: int) -> int:
    size = load_library().tg_select_topk_workspace_size(int(n))
    _need(size >= 0, "invalid select size")
    return size


def tg_select_topk_ws(g: torch.Tensor, k: int, q_len: int, idx: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """tg_select_topk spread over several workgroups, with a caller workspace."""
    lib = load_library()
    _need(g.dim() == 1 and g.dtype == torch.float32 and g.is_contiguous(), "g must be contiguous fp32 [n]")
    n = g.shape[0]
    kept = min(int(k), n)
    if idx is None:
        idx = torch.empty(kept, dtype=torch.int32, device=g.device)
    _vec(idx, kept, torch.int32, "idx")
    need = tg_select_topk_workspace_size(n)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=g.device)
    _need(workspace.is_contiguous(), "workspace must be contiguous")
    _check("tg_select_topk_ws",
           lib.tg_select_topk_ws(_ptr(g), n, int(k), int(q_len), _ptr(idx), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(g)))
    return idx


def tg_select_topk_varlen(g: torch.Tensor, cu_seqlens: torch.Tensor, q_lens: torch.Tensor, max_seqlen: int,
                          k: int, total_kept: int, idx_local: Optional[torch.Tensor] = None,
                          cu_kept: Optional[torch.Tensor] = None):
    """Per-prompt selection over a packed score vector; returns (idx_local, cu_kept).

    The kernel writes sum_b min(k, N_b) indices, which the host cannot know
    without reading cu_seqlens; idx_local is therefore sized for the bound
    min(batch * k, len(g)) (every prompt keeps at most k of its own tokens)."""
    lib = load_library()
    _need(g.dim() == 1 and g.dtype == torch.float32 and g.is_contiguous(), "g must be contiguous fp32 [total]")
    batch = cu_seqlens.numel() - 1
    _need(batch >= 0, "cu_seqlens needs batch + 1 entries")
    _vec(cu_seqlens, batch + 1, torch.int32, "cu_seqlens")
    _vec(q_lens, batch, torch.int32, "q_lens")
    bound = min(batch * max(int(k), 0), g.numel())
    _need(0 <= int(total_kept) <= bound, f"total_kept={total_kept} outside [0, {bound}]")
    if idx_local is None:
        idx_local = torch.empty(max(bound, 1), dtype=torch.int32, device=g.device)
    if cu_kept is None:
        cu_kept = torch.empty(batch + 1, dtype=torch.int32, device=g.device)
    _vec(idx_local, bound, torch.int32, "idx_local")
    _vec(cu_kept, batch + 1, torch.int32, "cu_kept")
    _check("tg_select_topk_varlen",
           lib.tg_select_topk_varlen(_ptr(g), _ptr(cu_seqlens), _ptr(q_lens), batch, int(max_seqlen), int(k),
                                     _ptr(idx_local), _ptr(cu_kept), _stream(g)))
    return idx_local[:total_kept], cu_kept


def tg_gather(h: torch.Tensor, g: Optional[torch.Tensor], idx: torch.Tensor, h_out: Optional[torch.Tensor] = None,
              g_out: Optional[torch.Tensor] = None, pos_out: Optional[torch.Tensor] = None):
    """(h[idx], g[idx], idx) as new tensors (or into the given ones)."""
    lib = load_library()
    _need(h.dim() == 2 and h.stride(1) == 1, "h must be [n, d] with unit column stride")
    n, d = h.shape
    nk = idx.numel()
    _vec(idx, nk, torch.int32, "idx")
    _vec(g, n, torch.float32, "g")
    if h_out is None:
        h_out = torch.empty(nk, d, dtype=h.dtype, device=h.device)
    if g is not None and g_out is None:
        g_out = torch.empty(nk, dtype=torch.float32, device=h.device)
    if pos_out is None:
        pos_out = torch.empty(nk, dtype=torch.int32, device=h.device)
    _like(h_out, (nk, d), h.dtype, "h_out")
    _vec(g_out, nk, torch.float32, "g_out")
    _vec(pos_out, nk, torch.int32, "pos_out")
    _check("tg_gather", lib.tg_gather(_dtype_code(h), n, nk, d, _ptr(idx), _ptr(h), h.stride(0), _ptr(g),
                                      _ptr(h_out), _ptr(g_out), _ptr(pos_out), _stream(h)))
    return h_out, g_out, pos_out


def tg_gather_varlen(h: torch.Tensor, g: Optional[torch.Tensor], idx_local: torch.Tensor, cu_seqlens: torch.Tensor,
                     cu_kept: torch.Tensor, max_kept: int, h_out=None, g_out=None, pos_out=None):
    lib = load_library()
    _need(h.dim() == 2 and h.stride(1) == 1, "h must be [n, d] with unit column stride")
    n, d = h.shape
    nk = idx_local.numel()
    batch = cu_seqlens.numel() - 1
    _vec(idx_local, nk, torch.int32, "idx_local")
    _vec(cu_seqlens, batch + 1, torch.int32, "cu_seqlens")
    _vec(cu_kept, batch + 1, torch.int32, "cu_kept")
    _vec(g, n, torch.float32, "g")
    if h_out is None:
        h_out = torch.empty(nk, d, dtype=h.dtype, device=h.device)
    if g is not None and g_out is None:
        g_out = torch.empty(nk, dtype=torch.float32, device=h.device)
    if pos_out is None:
        pos_out = torch.empty(nk, dtype=torch.int32, device=h.device)
    _like(h_out, (nk, d), h.dtype, "h_out")
    _vec(g_out, nk, torch.float32, "g_out")
    _vec(pos_out, nk, torch.int32, "pos_out")
    _check("tg_gather_varlen",
           lib.tg_gather_varlen(_dtype_code(h), _ptr(cu_seqlens), _ptr(cu_kept), batch, int(max_kept), d,
                                _ptr(idx_local), _ptr(h), h.stride(0), _ptr(g), _ptr(h_out), _ptr(g_out),
                                _ptr(pos_out), _stream(h)))
    return h_out, g_out, pos_out


def tg_rope_table(max_pos: int, dh: int, base: float, device, out: Optional[torch.Tensor] = None):
    """cos/sin table [max_pos, dh] fp32 (cos | sin halves), built on the device in fp64."""
    lib = load_library()
    if out is None:
        out = torch.empty(max_pos, dh, dtype=torch.float32, device=device)
    _check("tg_rope_table", lib.tg_rope_table(_ptr(out), int(max_pos), int(dh), float(base), _stream(out)))
    return out


def tg_rope_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, cos_sin: torch.Tensor,
               k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None):
    """Rotates q in place; returns (q, k_cache, v_cache)."""
    lib = load_library()
    _need(q.dim() == 3, "q must be [n, hq, dh]")
    n, hq, dh = q.shape
    hkv = k.shape[1] if k.dim() == 3 else -1
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share a dtype")
    _need(k.dim() == 3 and tuple(k.shape) == (n, hkv, dh) and tuple(v.shape) == (n, hkv, dh),
          "k and v must be [n, hkv, dh]")
    _vec(pos, n, torch.int32, "pos")
    _need(cos_sin.dim() == 2 and cos_sin.shape[1] == dh and cos_sin.dtype == torch.float32 and
          cos_sin.is_contiguous(), "cos_sin must be a contiguous fp32 [max_pos, dh] table")
    if k_cache is None:
        k_cache = torch.empty_like(k)
    if v_cache is None:
        v_cache = torch.empty_like(v)
    _like(k_cache, k.shape, k.dtype, "k_cache")
    _like(v_cache, v.shape, v.dtype, "v_cache")
    _check("tg_rope_kv", lib.tg_rope_kv(_dtype_code(q), n, hq, hkv, dh, _ptr(pos), _ptr(cos_sin),
                                        cos_sin.shape[0], _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache),
                                        _ptr(v_cache), _stream(q)))
    return q, k_cache, v_cache


def _check_attn_operands(q, k, v, g, pos, head_gain, rows):
    _need(q.dim() == 3 and k.dim() == 3, "q must be [n, hq, dh] and k, v [n, hkv, dh]")
    n, hq, dh = q.shape
    hkv = k.shape[1]
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share a dtype")
    _need(tuple(k.shape) == (n, hkv, dh) and tuple(v.shape) == (n, hkv, dh), "k and v must be [n, hkv, dh]")
    _vec(g, rows, torch.float32, "g")
    _vec(pos, rows, torch.int32, "pos")
    _need(pos is not None, "pos is required")
    _vec(head_gain, hq, torch.float32, "head_gain")
    return n, hq, hkv, dh


def _attn_outputs(q, o, lse, want_lse, hq, n):
    if o is None:
        o = torch.empty_like(q)
    _like(o, q.shape, q.dtype, "o")
    if want_lse and lse is None:
        lse = torch.empty(hq, n, dtype=torch.float32, device=q.device)
    if lse is not None:
        _like(lse, (hq, n), torch.float32, "lse")
    return o, lse


def tg_gated_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor], pos: torch.Tensor,
                  scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                  head_gain: Optional[torch.Tensor] = None):
    """Token-gated causal GQA attention; returns o (and lse [hq, n] if requested).

    g=None: no gate (plain causal attention).  head_gain: [hq] fp32 multiplier
    of the gate bias per query head (tg_gated_attn_ex)."""
    lib = load_library()
    n, hq, hkv, dh = _check_attn_operands(q, k, v, g, pos, head_gain, q.shape[0] if q.dim() == 3 else 0)
    if scale is None:
        scale = dh ** -0.5
    o, lse = _attn_outputs(q, o, lse, want_lse, hq, n)
    if g is None or head_gain is not None:
        _check("tg_gated_attn_ex",
               lib.tg_gated_attn_ex(_dtype_code(q), None, 1, n, n, hq, hkv, dh, float(scale), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(g), _ptr(head_gain), _ptr(pos), _ptr(o), _ptr(lse), _stream(q)))
    else:
        _check("tg_gated_attn", lib.tg_gated_attn(_dtype_code(q), n, hq, hkv, dh, float(scale), _ptr(q), _ptr(k),
                                                  _ptr(v), _ptr(g), _ptr(pos), _ptr(o), _ptr(lse), _stream(q)))
    return (o, lse) if (want_lse or lse is not None) else o


def tg_gated_attn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                         pos: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                         scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                         head_gain: Optional[torch.Tensor] = None):
    """Packed ragged batch.  max_seqlen must bound every prompt's row count
    (cu_seqlens stays on the device, so the host does not check it)."""
    lib = load_library()
    total, hq, hkv, dh = _check_attn_operands(q, k, v, g, pos, head_gain, q.shape[0] if q.dim() == 3 else 0)
    batch = cu_seqlens.numel() - 1
    _vec(cu_seqlens, batch + 1, torch.int32, "cu_seqlens")
    _need(0 <= int(max_seqlen) and (batch == 0 or int(max_seqlen) <= total or total == 0),
          "max_seqlen must lie in [0, total rows]")
    if scale is None:
        scale = dh ** -0.5
    o, lse = _attn_outputs(q, o, lse, want_lse, hq, total)
    if g is None or head_gain is not None:
        _check("tg_gated_attn_ex",
               lib.tg_gated_attn_ex(_dtype_code(q), _ptr(cu_seqlens), batch, int(max_seqlen), total, hq, hkv, dh,
                                    float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(head_gain), _ptr(pos),
                                    _ptr(o), _ptr(lse), _stream(q)))
    else:
        _check("tg_gated_attn_varlen",
               lib.tg_gated_attn_varlen(_dtype_code(q), _ptr(cu_seqlens), batch, int(max_seqlen), total, hq, hkv,
                                        dh, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(pos), _ptr(o),
                                        _ptr(lse), _stream(q)))
    return (o, lse) if (want_lse or lse is not None) else o


def tg_decode_attn_workspace_size(batch: int, max_seqlen: int, hq: int, hkv: int, dh: int) -> int:
    n = load_library().tg_decode_attn_workspace_size(batch, int(max_seqlen), hq, hkv, dh)
    _need(n >= 0, "invalid decode sizes")
    return n


def tg_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, g: Optional[torch.Tensor],
                   cu_seqlens: torch.Tensor, max_seqlen: int, scale: Optional[float] = None,
                   head_gain: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                   workspace: Optional[torch.Tensor] = None):
    """One new query per sequence over its packed cache; q [B, hq, dh]."""
    lib = load_library()
    batch, hq, dh = q.shape
    hkv = k_cache.shape[1]
    _vec(cu_seqlens, batch + 1, torch.int32, "cu_seqlens")
    _need(cu_seqlens.numel() == batch + 1, "cu_seqlens is int32 [B + 1]")
    _need(q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous(), "q and caches contiguous")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and the caches share a dtype")
    _need(k_cache.dim() == 3 and k_cache.shape[2] == dh and tuple(v_cache.shape) == tuple(k_cache.shape),
          "k_cache and v_cache must be [total, hkv, dh]")
    _vec(g, k_cache.shape[0], torch.float32, "g")
    _vec(head_gain, hq, torch.float32, "head_gain")
    if scale is None:
        scale = dh ** -0.5
    if o is None:
        o = torch.empty_like(q)
    _like(o, q.shape, q.dtype, "o")
    if want_lse and lse is None:
        lse = torch.empty(batch, hq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _like(lse, (batch, hq), torch.float32, "lse")
    need = tg_decode_attn_workspace_size(batch, max_seqlen, hq, hkv, dh)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("tg_decode_attn",
           lib.tg_decode_attn(_dtype_code(q), _ptr(cu_seqlens), batch, int(max_seqlen), hq, hkv, dh, float(scale),
                              _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(g), _ptr(head_gain), _ptr(o), _ptr(lse),
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, lse) if (want_lse or lse is not None) else o


def tg_decode_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, g: Optional[torch.Tensor],
                           cu_seqlens: torch.Tensor, max_seqlen: int, o: torch.Tensor,
                           lse: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                           head_gain: Optional[torch.Tensor] = None):
    """tg_decode_attn with the library's static scratch instead of a workspace:
    the library allocates nothing (and neither does this wrapper: o, and lse
    if wanted, are the caller's).  Returns o."""
    lib = load_library()
    _need(q.dim() == 3, "q must be [B, hq, dh]")
    batch, hq, dh = q.shape
    hkv = k_cache.shape[1] if k_cache.dim() == 3 else -1
    _vec(cu_seqlens, batch + 1, torch.int32, "cu_seqlens")
    _need(cu_seqlens.numel() == batch + 1, "cu_seqlens is int32 [B + 1]")
    _need(q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous(), "q and caches contiguous")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and the caches share a dtype")
    _need(k_cache.dim() == 3 and k_cache.shape[2] == dh and tuple(v_cache.shape) == tuple(k_cache.shape),
          "k_cache and v_cache must be [total, hkv, dh]")
    _vec(g, k_cache.shape[0], torch.float32, "g")
    _vec(head_gain, hq, torch.float32, "head_gain")
    _like(o, q.shape, q.dtype, "o")
    if lse is not None:
        _like(lse, (batch, hq), torch.float32, "lse")
    if scale is None:
        scale = dh ** -0.5
    _check("tg_decode_attn_noalloc",
           lib.tg_decode_attn_noalloc(_dtype_code(q), _ptr(cu_seqlens), batch, int(max_seqlen), hq, hkv, dh,
                                      float(scale), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(g), _ptr(head_gain),
                                      _ptr(o), _ptr(lse), _stream(q)))
    return o


def tg_linear(x: torch.Tensor, w: torch.Tensor, residual: Optional[torch.Tensor] = None,
              y: Optional[torch.Tensor] = None):
    """y = x W^T (+ residual); x [M, K], w [N, K] (row strides taken from the tensors)."""
    lib = load_library()
    m, k = x.shape
    n = w.shape[0]
    _need(w.shape[1] == k and x.stride(1) == 1 and w.stride(1) == 1, "x [M, K] and w [N, K], rows contiguous")
    if y is None:
        y = torch.empty(m, n, dtype=x.dtype, device=x.device)
    _need(y.stride(1) == 1 and (residual is None or residual.stride(1) == 1), "rows of y and residual contiguous")
    _check("tg_linear",
           lib.tg_linear(_dtype_code(x), m, n, k, _ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(residual),
                         residual.stride(0) if residual is not None else 0, _ptr(y), y.stride(0), _stream(x)))
    return y


def tg_swiglu(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, y: Optional[torch.Tensor] = None):
    """y = SiLU(x Wg^T) * (x Wu^T); x [M, K], w_gate and w_up [F, K] with the same row stride."""
    lib = load_library()
    m, k = x.shape
    f = w_gate.shape[0]
    _need(tuple(w_up.shape) == tuple(w_gate.shape) and w_up.stride(0) == w_gate.stride(0), "w_gate, w_up alike")
    _need(x.stride(1) == 1 and w_gate.stride(1) == 1 and w_up.stride(1) == 1, "rows contiguous")
    if y is None:
        y = torch.empty(m, f, dtype=x.dtype, device=x.device)
    _check("tg_swiglu",
           lib.tg_swiglu(_dtype_code(x), m, f, k, _ptr(x), x.stride(0), _ptr(w_gate), _ptr(w_up), w_gate.stride(0),
                         _ptr(y), y.stride(0), _stream(x)))
    return y


def tg_qkv_proj(x: torch.Tensor, w_qkv: torch.Tensor, hq: int, hkv: int, dh: int,
                q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None):
    """q [M, hq, dh], k and v [M, hkv, dh] from one product with w_qkv [(hq + 2 hkv) dh, K]."""
    lib = load_library()
    m, kin = x.shape
    _need(tuple(w_qkv.shape) == ((hq + 2 * hkv) * dh, kin) and x.stride(1) == 1 and w_qkv.stride(1) == 1,
          "x [M, K], w_qkv [(hq + 2 hkv) dh, K]")
    q = torch.empty(m, hq, dh, dtype=x.dtype, device=x.device) if q is None else q
    k = torch.empty(m, hkv, dh, dtype=x.dtype, device=x.device) if k is None else k
    v = torch.empty(m, hkv, dh, dtype=x.dtype, device=x.device) if v is None else v
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v contiguous")
    _check("tg_qkv_proj",
           lib.tg_qkv_proj(_dtype_code(x), m, hq, hkv, dh, kin, _ptr(x), x.stride(0), _ptr(w_qkv), w_qkv.stride(0),
                           _ptr(q), _ptr(k), _ptr(v), _stream(x)))
    return q, k, v


def tg_check_positions(pos: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                       first_bad: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device int32 [1]: the smallest row whose position breaks the strictly
    increasing order within its sequence (or is negative), else len(pos)."""
    lib = load_library()
    _need(pos.dtype == torch.int32, "pos is int32")
    if first_bad is None:
        first_bad = torch.empty(1, dtype=torch.int32, device=pos.device)
    batch = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _check("tg_check_positions",
           lib.tg_check_positions(_ptr(pos), pos.numel(), _ptr(cu_seqlens), batch, _ptr(first_bad), _stream(pos)))
    return first_bad
