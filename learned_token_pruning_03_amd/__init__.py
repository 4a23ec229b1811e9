"""TokenGate gated-prefill hot path for AMD Instinct MI355X (gfx950).

The computation lives in ``libtokengate.so`` (hand-written HIP kernels behind
the C ABI of ``include/tokengate.h``); this package holds its ctypes binding
(``binding``), the in-tree build (``build``) and seeded synthetic workloads
(``workloads``).
"""
from .binding import (  # noqa: F401
    LIB_PATH,
    SIGNATURES,
    TG_BF16,
    TG_ERR_HIP,
    TG_ERR_INVALID_ARG,
    TG_ERR_UNSUPPORTED,
    TG_ERR_WORKSPACE,
    TG_FP32,
    TG_OK,
    TokenGateError,
    load_library,
    status_string,
    tg_check_positions,
    tg_decode_attn,
    tg_decode_attn_noalloc,
    tg_decode_attn_workspace_size,
    select_workspace,
    tg_gate_score,
    tg_gate_select,
    tg_gate_select_gather,
    tg_gated_attn,
    tg_gated_attn_varlen,
    tg_gather,
    tg_gather_varlen,
    tg_linear,
    tg_qkv_proj,
    tg_rope_kv,
    tg_rope_table,
    tg_select_topk,
    tg_select_topk_varlen,
    tg_select_topk_workspace_size,
    tg_select_topk_ws,
    tg_swiglu,
)
