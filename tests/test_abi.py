"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

import learned_token_pruning_03_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TG_API\s+[\w\s\*]+?\b(tg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tg.load_library()


def test_header_declares_the_expected_entry_points():
    syms = declared_symbols()
    for name in ("tg_gate_score", "tg_gate_select", "tg_gate_select_gather", "tg_select_topk", "tg_select_topk_varlen", "tg_select_topk_workspace_size",
                 "tg_select_topk_ws", "tg_gather", "tg_gather_varlen",
                 "tg_rope_table", "tg_rope_kv", "tg_gated_attn", "tg_gated_attn_varlen", "tg_gated_attn_ex",
                 "tg_decode_attn_workspace_size", "tg_decode_attn",
                 "tg_linear", "tg_swiglu", "tg_qkv_proj", "tg_check_positions",
                 "tg_status_string",
                 "tg_last_error", "tg_abi_version"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in tg.SIGNATURES, f"binding lacks a signature for {name}"


def test_status_strings_and_version(lib):
    assert lib.tg_abi_version() == 1
    assert tg.status_string(0) == "TG_OK"
    assert tg.status_string(1) == "TG_ERR_INVALID_ARG"
    assert tg.status_string(3) == "TG_ERR_WORKSPACE"
    assert tg.status_string(4) == "TG_ERR_HIP"
    assert tg.status_string(99) == "TG_UNKNOWN_STATUS"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _err(lib):
    return lib.tg_last_error().decode()


def test_select_rejects_question_longer_than_budget(lib):
    assert lib.tg_select_topk(FAKE, 100, 10, 11, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert "q_len" in _err(lib)
    assert lib.tg_select_topk(FAKE, 5, 100, 6, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_select_topk(FAKE, -1, 10, 0, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_select_topk(None, 10, 5, 1, FAKE, None) == tg.TG_ERR_INVALID_ARG


def test_zero_sized_calls_are_noops(lib):
    assert lib.tg_select_topk(None, 0, 0, 0, None, None) == tg.TG_OK
    assert lib.tg_gate_score(tg.TG_BF16, 0, 64, 256, None, 64, None, None, None, 0.0, None, None, None) == tg.TG_OK
    assert lib.tg_gather(tg.TG_BF16, 10, 0, 64, None, None, 64, None, None, None, None, None) == tg.TG_OK
    assert lib.tg_gated_attn(tg.TG_BF16, 0, 16, 8, 128, 0.1, None, None, None, None, None, None, None,
                             None) == tg.TG_OK


def test_gate_rejects_unsupported_shapes(lib):
    args = (FAKE, 2048, FAKE, None, FAKE, 0.0, FAKE, None, None)
    assert lib.tg_gate_score(tg.TG_BF16, 10, 2000, 256, *args) == tg.TG_ERR_UNSUPPORTED
    assert lib.tg_gate_score(tg.TG_BF16, 10, 2048, 100, *args) == tg.TG_ERR_UNSUPPORTED
    assert lib.tg_gate_score(7, 10, 2048, 256, *args) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_gate_score(tg.TG_BF16, 10, 2048, 256, FAKE, 1000, FAKE, None, FAKE, 0.0, FAKE, None,
                             None) == tg.TG_ERR_INVALID_ARG  # ld_h < d
    assert lib.tg_gate_score(tg.TG_BF16, 10, 2048, 256, FAKE + 2, 2048, FAKE, None, FAKE, 0.0, FAKE, None,
                             None) == tg.TG_ERR_INVALID_ARG  # misaligned h


def test_attn_rejects_bad_heads_and_head_dim(lib):
    p = [FAKE] * 5
    assert lib.tg_gated_attn(tg.TG_BF16, 16, 6, 4, 128, 0.1, *p, FAKE, None, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_gated_attn(tg.TG_BF16, 16, 16, 8, 96, 0.1, *p, FAKE, None, None) == tg.TG_ERR_UNSUPPORTED
    assert lib.tg_gated_attn(tg.TG_BF16, 16, 16, 8, 128, 0.0, *p, FAKE, None, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_gated_attn(tg.TG_BF16, 16, 16, 8, 128, 0.1, None, *p[1:], FAKE, None,
                             None) == tg.TG_ERR_INVALID_ARG


def test_attn_ex_validation_without_a_gpu(lib):
    # tg_gated_attn_ex(dtype, cu, batch, max_seqlen, total, hq, hkv, dh, scale, q, k, v, g, head_gain, pos, o,
    #                  lse, stream); g and head_gain may be NULL, the tensors may not.
    assert lib.tg_gated_attn_ex(tg.TG_BF16, None, 1, 16, 0, 16, 8, 128, 0.1, None, None, None, None, None, None,
                                None, None, None) == tg.TG_OK  # nothing to do
    assert lib.tg_gated_attn_ex(tg.TG_BF16, None, 1, 16, 16, 6, 4, 128, 0.1, FAKE, FAKE, FAKE, None, None, FAKE,
                                FAKE, None, None) == tg.TG_ERR_INVALID_ARG  # hq not a multiple of hkv
    assert lib.tg_gated_attn_ex(tg.TG_BF16, None, 1, 16, 16, 16, 8, 96, 0.1, FAKE, FAKE, FAKE, None, None, FAKE,
                                FAKE, None, None) == tg.TG_ERR_UNSUPPORTED  # head dim
    assert lib.tg_gated_attn_ex(tg.TG_BF16, None, 1, 16, 16, 16, 8, 128, 0.1, FAKE, FAKE, FAKE, None, None, None,
                                FAKE, None, None) == tg.TG_ERR_INVALID_ARG  # NULL pos
    assert lib.tg_gated_attn_ex(tg.TG_BF16, None, 1, 16, -1, 16, 8, 128, 0.1, FAKE, FAKE, FAKE, None, None, FAKE,
                                FAKE, None, None) == tg.TG_ERR_INVALID_ARG  # negative total


def test_decode_validation_without_a_gpu(lib):
    # tg_decode_attn(dtype, cu, batch, max_seqlen, hq, hkv, dh, scale, q, k_cache, v_cache, g, head_gain, o, lse,
    #                workspace, workspace_bytes, stream)
    ws = lib.tg_decode_attn_workspace_size(4, 5000, 16, 8, 128)
    assert ws > 0 and ws % 16 == 0
    assert lib.tg_decode_attn_workspace_size(4, 5000, 16, 8, 96) == -1
    assert lib.tg_decode_attn_workspace_size(4, 5000, 6, 4, 128) == -1
    assert lib.tg_decode_attn_workspace_size(-1, 5000, 16, 8, 128) == -1
    assert lib.tg_decode_attn_workspace_size(4, 0, 16, 8, 128) > 0  # empty caches still write o and lse

    def call(batch=4, max_seqlen=5000, hq=16, hkv=8, dh=128, scale=0.1, q=FAKE, ws_bytes=ws, cu=FAKE):
        return lib.tg_decode_attn(tg.TG_BF16, cu, batch, max_seqlen, hq, hkv, dh, scale, q, FAKE, FAKE, None,
                                  None, FAKE, None, FAKE, ws_bytes, None)

    assert call(batch=0) == tg.TG_OK  # nothing to do
    assert call(hq=24, hkv=8) == tg.TG_ERR_UNSUPPORTED  # three query heads per KV head
    assert call(hq=32, hkv=2) == tg.TG_ERR_UNSUPPORTED  # sixteen
    assert call(dh=96) == tg.TG_ERR_UNSUPPORTED
    assert call(hq=6, hkv=4) == tg.TG_ERR_INVALID_ARG
    assert call(scale=0.0) == tg.TG_ERR_INVALID_ARG
    assert call(q=None) == tg.TG_ERR_INVALID_ARG
    assert call(cu=None) == tg.TG_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 4) == tg.TG_ERR_WORKSPACE
    assert b"workspace" in lib.tg_last_error()
    assert call(max_seqlen=-1) == tg.TG_ERR_INVALID_ARG
    big = lib.tg_decode_attn_workspace_size(70000, 5000, 16, 8, 128)
    assert call(batch=70000, ws_bytes=big) == tg.TG_ERR_UNSUPPORTED  # one grid row per sequence


def test_dense_validation_without_a_gpu(lib):
    # tg_linear(dtype, m, n, k, x, ld_x, w, ld_w, residual, ld_r, y, ld_y, stream)
    def lin(dtype=tg.TG_BF16, m=64, n=256, k=64, x=FAKE, ld_x=64, w=FAKE, ld_w=64, r=None, ld_r=0, ld_y=256):
        return lib.tg_linear(dtype, m, n, k, x, ld_x, w, ld_w, r, ld_r, FAKE, ld_y, None)

    assert lin(m=0) == tg.TG_OK
    assert lin(dtype=tg.TG_FP32) == tg.TG_ERR_UNSUPPORTED
    assert lin(n=320) == tg.TG_ERR_UNSUPPORTED
    assert lin(k=48, ld_x=48, ld_w=48) == tg.TG_ERR_UNSUPPORTED
    assert lin(ld_x=32) == tg.TG_ERR_INVALID_ARG
    assert lin(ld_x=68) == tg.TG_ERR_INVALID_ARG  # rows not 16-byte aligned
    assert lin(ld_y=128) == tg.TG_ERR_INVALID_ARG
    assert lin(x=None) == tg.TG_ERR_INVALID_ARG
    assert lin(x=FAKE + 8) == tg.TG_ERR_INVALID_ARG
    assert lin(r=FAKE, ld_r=100) == tg.TG_ERR_INVALID_ARG
    assert lin(m=-1) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_linear(tg.TG_BF16, 64, 256, 64, FAKE, 64, FAKE, 64, FAKE + 4096, 512, FAKE + 4096, 256,
                         None) == tg.TG_ERR_INVALID_ARG  # in-place residual with another stride
    # tg_swiglu(dtype, m, f, k, x, ld_x, w_gate, w_up, ld_w, y, ld_y, stream)
    assert lib.tg_swiglu(tg.TG_BF16, 0, 128, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 128, None) == tg.TG_OK
    assert lib.tg_swiglu(tg.TG_BF16, 8, 192, 64, FAKE, 64, FAKE, FAKE, 64, FAKE, 192, None) == tg.TG_ERR_UNSUPPORTED
    assert lib.tg_swiglu(tg.TG_BF16, 8, 128, 64, FAKE, 64, FAKE, None, 64, FAKE, 128, None) == tg.TG_ERR_INVALID_ARG
    # tg_qkv_proj(dtype, m, hq, hkv, dh, k, x, ld_x, w_qkv, ld_w, q, k_out, v_out, stream)
    assert lib.tg_qkv_proj(tg.TG_BF16, 0, 16, 8, 128, 64, FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, None) == tg.TG_OK
    assert lib.tg_qkv_proj(tg.TG_BF16, 8, 4, 2, 64, 64, FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE,
                           None) == tg.TG_ERR_UNSUPPORTED  # hkv*dh = 128
    assert lib.tg_qkv_proj(tg.TG_BF16, 8, 16, 8, 128, 64, FAKE, 64, FAKE, 64, FAKE, None, FAKE,
                           None) == tg.TG_ERR_INVALID_ARG


def test_check_positions_validation_without_a_gpu(lib):
    # tg_check_positions(pos, total, cu_seqlens, batch, first_bad, stream)
    assert lib.tg_check_positions(FAKE, 10, None, 0, None, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_check_positions(None, 10, None, 0, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_check_positions(FAKE, -1, None, 0, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_check_positions(FAKE, 10, FAKE, -2, FAKE, None) == tg.TG_ERR_INVALID_ARG


def test_gather_and_rope_validation(lib):
    assert lib.tg_gather(tg.TG_BF16, 10, 4, 12, FAKE, FAKE, 12, FAKE, FAKE, FAKE, FAKE,
                         None) == tg.TG_ERR_UNSUPPORTED  # 24-byte rows
    assert lib.tg_gather(tg.TG_BF16, 10, 4, 64, FAKE, FAKE, 64, FAKE, FAKE, None, FAKE,
                         None) == tg.TG_ERR_INVALID_ARG  # g without g_out
    assert lib.tg_rope_kv(tg.TG_BF16, 4, 16, 8, 100, FAKE, FAKE, 10, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None) == tg.TG_ERR_UNSUPPORTED
    assert lib.tg_rope_table(FAKE, 10, 7, 1e6, None) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_rope_table(FAKE, 10, 8, 0.5, None) == tg.TG_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        tg.tg_select_topk(torch.zeros(10), 5, 1)


def test_grids_beyond_one_dispatch_are_refused_before_any_hip_call(lib):
    """A dispatch counts work-items in 32 bits in x and 65535 workgroups in y and
    z; sizes that fit in memory can still exceed that, and must be refused on the
    host (TG_ERR_UNSUPPORTED), not launched with a truncated grid."""
    U = tg.TG_ERR_UNSUPPORTED
    # gather: one wave per row, 2^26 rows of 16 bytes (1 GiB) -> 2^32 work-items
    assert lib.tg_gather(tg.TG_BF16, 1 << 27, 1 << 26, 8, FAKE, FAKE, 8, None, FAKE, None, None, None) == U
    assert b"launch grid" in lib.tg_last_error()
    # rope_kv: one 256-thread workgroup per kept token
    assert lib.tg_rope_kv(tg.TG_BF16, 1 << 24, 1, 1, 16, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == U
    # rope_table: one work-item per (position, frequency)
    assert lib.tg_rope_table(FAKE, 1 << 26, 128, 10000.0, None) == U
    # fp32 gate: four rows per 256-thread workgroup
    assert lib.tg_gate_score(tg.TG_FP32, 1 << 26, 4, 4, FAKE, 4, FAKE, None, FAKE, 0.0, FAKE, None, None) == U
    # ragged select: one 1024-thread workgroup per prompt
    assert lib.tg_select_topk_varlen(FAKE, FAKE, FAKE, 1 << 22, 1, 1, FAKE, FAKE, None) == U
    # fp32 attention: query heads index the grid's y dimension
    assert lib.tg_gated_attn(tg.TG_FP32, 16, 70000, 70000, 64, 0.1, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                             None) == U
    # decode: KV heads index the grid's y dimension
    ws = lib.tg_decode_attn_workspace_size(1, 64, 70000, 70000, 64)
    assert ws > 0
    assert lib.tg_decode_attn(tg.TG_BF16, FAKE, 1, 64, 70000, 70000, 64, 0.1, FAKE, FAKE, FAKE, None, None, FAKE,
                              None, FAKE, ws, None) == U
    # the same gather with nothing to copy is a no-op, not a refusal
    assert lib.tg_gather(tg.TG_BF16, 1 << 27, 0, 8, FAKE, FAKE, 8, None, FAKE, None, None, None) == tg.TG_OK


def test_select_ws_validation_without_a_gpu(lib):
    ws = lib.tg_select_topk_workspace_size(32768)
    # an 11-bit histogram, an arrival counter, T, need and the item count; two counts per 64-token
    # chunk; then up to one copy item per chunk plus one per 8 tokens; then, from a 64-word
    # boundary, one order key per token, padded to a whole number of 256-key blocks
    def words(n):
        chunks = -(-n // 64)
        head = 2048 + 64 + 2 * chunks + chunks + -(-n // 8)
        return -(-head // 64) * 64 + -(-n // 256) * 256
    assert ws == 4 * words(32768) == 4 * (7744 + 32768)
    assert lib.tg_select_topk_workspace_size(100) == 4 * words(100) == 4 * (2176 + 256)
    assert lib.tg_select_topk_workspace_size(131072) == 4 * words(131072)
    assert lib.tg_select_topk_workspace_size(-1) == -1
    ok = tg.TG_ERR_INVALID_ARG
    assert lib.tg_select_topk_ws(FAKE, 32768, 4096, 64, FAKE, FAKE, ws - 4, None) == tg.TG_ERR_WORKSPACE
    assert lib.tg_select_topk_ws(FAKE, 32768, 4096, 64, FAKE, None, ws, None) == ok  # NULL workspace
    assert lib.tg_select_topk_ws(FAKE, 32768, 4096, 64, FAKE, FAKE + 4, ws, None) == ok  # misaligned
    assert lib.tg_select_topk_ws(FAKE, 32768, 10, 11, FAKE, FAKE, ws, None) == ok  # q_len > budget
    assert lib.tg_select_topk_ws(FAKE, 0, 10, 0, FAKE, None, 0, None) == tg.TG_OK  # empty: no-op


def test_gate_select_validation_without_a_gpu(lib):
    """The fused gate + select checks the gate's arguments, the selection's and
    the workspace's before any HIP call."""
    ws = lib.tg_select_topk_workspace_size(32768)
    E, W, U = tg.TG_ERR_INVALID_ARG, tg.TG_ERR_WORKSPACE, tg.TG_ERR_UNSUPPORTED

    def call(dt=tg.TG_BF16, n=32768, d=2048, hidden=256, h=FAKE, ld=2048, w1=FAKE, w2=FAKE, k=4096, q=64, g=FAKE,
             idx=FAKE, wsp=FAKE, wsb=ws):
        return lib.tg_gate_select(dt, n, d, hidden, h, ld, w1, None, w2, 0.0, k, q, g, None, idx, wsp, wsb, None)

    assert call(q=4097) == E and "q_len" in _err(lib)
    assert call(k=-1) == E
    assert call(wsb=ws - 4) == W
    assert call(wsp=None) == E
    assert call(wsp=FAKE + 4) == E
    assert call(idx=None) == E
    assert call(g=None) == E
    assert call(hidden=100) == U
    assert call(d=100) == U
    assert call(h=FAKE + 2) == E
    assert call(n=0, h=None, w1=None, w2=None, g=None, idx=None, wsp=None, k=0, q=0) == tg.TG_OK  # empty: no-op
    # the gathering form also needs an aligned h_out
    gsg = lib.tg_gate_select_gather
    assert gsg(tg.TG_BF16, 32768, 2048, 256, FAKE, 2048, FAKE, None, FAKE, 0.0, 4096, 64, FAKE, None, FAKE, None,
               None, None, FAKE, ws, None) == E
    assert gsg(tg.TG_BF16, 32768, 2048, 256, FAKE, 2048, FAKE, None, FAKE, 0.0, 4096, 64, FAKE, None, FAKE, FAKE + 4,
               None, None, FAKE, ws, None) == E
    assert gsg(tg.TG_BF16, 32768, 2048, 256, FAKE, 2048, FAKE, None, FAKE, 0.0, 4096, 64, FAKE, None, FAKE, FAKE,
               None, None, FAKE, ws - 4, None) == W


def test_binding_rejects_mismatched_buffers_before_any_call():
    """The C ABI takes no buffer lengths, so the binding checks dtypes, shapes
    and sizes itself; a mismatch raises ValueError before the library is
    called (CPU tensors suffice: the checks come before the device check)."""
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    n, hq, hkv, dh = 8, 4, 2, 64
    q = torch.zeros(n, hq, dh, dtype=bf)
    k = torch.zeros(n, hkv, dh, dtype=bf)
    pos = torch.arange(n, dtype=i32)
    g = torch.ones(n, dtype=f32)
    cases = [
        lambda: tg.tg_gated_attn(q.float(), k, k, g, pos),                       # q fp32, k bf16
        lambda: tg.tg_gated_attn(q, k[:4], k[:4], g, pos),                       # k rows < q rows
        lambda: tg.tg_gated_attn(q, k, k, g[:4], pos),                           # g too short
        lambda: tg.tg_gated_attn(q, k, k, g, pos.long()),                        # pos not int32
        lambda: tg.tg_gated_attn(q, k, k, g, pos, o=torch.zeros(n, hq, dh, dtype=f32)),  # o dtype
        lambda: tg.tg_gated_attn(q, k, k, g, pos, lse=torch.zeros(hq, n - 1)),   # lse shape
        lambda: tg.tg_gated_attn(q, k, k, g, pos, head_gain=torch.ones(hq - 1)),  # gains per head
        lambda: tg.tg_gated_attn_varlen(q, k, k, g, pos, torch.tensor([0, 4, 8], dtype=torch.int64), 4),
        lambda: tg.tg_rope_kv(q, k, k, pos, torch.zeros(16, dh // 2)),           # table for another dh
        lambda: tg.tg_rope_kv(q, k, k, pos, torch.zeros(16, dh, dtype=torch.float64)),
        lambda: tg.tg_rope_kv(q, k, k.float(), pos, torch.zeros(16, dh)),        # v dtype
        lambda: tg.tg_rope_kv(q, k, k, pos[:4], torch.zeros(16, dh)),           # too few positions
        lambda: tg.tg_gather(torch.zeros(16, 64, dtype=bf), g, torch.arange(4)),  # idx int64
        lambda: tg.tg_gather(torch.zeros(16, 64, dtype=bf), g[:4], torch.arange(4, dtype=i32)),  # g < n rows
        lambda: tg.tg_gather(torch.zeros(16, 64, dtype=bf), None, torch.arange(4, dtype=i32),
                             h_out=torch.zeros(3, 64, dtype=bf)),               # h_out rows
        lambda: tg.tg_select_topk_varlen(torch.zeros(100), torch.tensor([0, 50, 100], dtype=i32),
                                         torch.tensor([1, 1], dtype=i32), 50, 10, 21),  # total_kept > 2 x 10
        lambda: tg.tg_select_topk_varlen(torch.zeros(100), torch.tensor([0, 50, 100], dtype=i32),
                                         torch.tensor([1, 1], dtype=i32), 50, 10, 20,
                                         idx_local=torch.zeros(19, dtype=i32)),  # idx_local too short
        lambda: tg.tg_select_topk(torch.zeros(10), 5, 1, idx=torch.zeros(4, dtype=i32)),
        lambda: tg.tg_decode_attn(q[:2], k, k, g[:4], torch.tensor([0, 4, 8], dtype=i32), 4),  # g < cache rows
        lambda: tg.tg_decode_attn(q[:2], k, k.float(), None, torch.tensor([0, 4, 8], dtype=i32), 4),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
            pytest.fail(f"case {i} was not refused")


def test_noalloc_decode_refuses_oversized_requests_without_a_gpu(lib):
    """The static-scratch decode checks its scratch need on the host, before any
    HIP call, and names the limit."""
    assert lib.tg_decode_attn_noalloc_max_bytes() == 16 << 20
    st = lib.tg_decode_attn_noalloc(tg.TG_BF16, FAKE, 64, 1 << 20, 16, 8, 128, 0.1, FAKE, FAKE, FAKE, None, None,
                                    FAKE, None, None)
    assert st == tg.TG_ERR_WORKSPACE
    assert "static scratch" in _err(lib)
    assert lib.tg_decode_attn_noalloc(tg.TG_BF16, FAKE, 0, 16, 16, 8, 128, 0.1, None, None, None, None, None, None,
                                      None, None) == tg.TG_OK  # empty batch: no-op
    assert lib.tg_decode_attn_noalloc(tg.TG_BF16, FAKE, 2, 16, 16, 8, 100, 0.1, FAKE, FAKE, FAKE, None, None, FAKE,
                                      None, None) == tg.TG_ERR_UNSUPPORTED  # dh
