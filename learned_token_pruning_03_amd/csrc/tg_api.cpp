// Host side of the C ABI declared in include/tokengate.h: argument validation
// (before any HIP call), dispatch to the kernel launchers, error reporting.
#include "tokengate.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tg_internal.h"

namespace {

thread_local char g_last_error[512] = "";

tg_status fail(tg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

tg_status ok() {
  g_last_error[0] = '\0';
  return TG_OK;
}

tg_status from_hip(hipError_t e, const char* what) {
  if (e == hipErrorInvalidConfiguration)  // refused by a launcher before any HIP call
    return fail(TG_ERR_UNSUPPORTED, "%s: launch grid beyond 2^32 work-items in x or 65535 blocks in y, z", what);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    return fail(TG_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  }
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(tg_dtype dt) { return dt == TG_BF16 ? 2 : 4; }

bool valid_dtype(tg_dtype dt) { return dt == TG_BF16 || dt == TG_FP32; }

constexpr int64_t kMaxI32 = 2147483647LL;
constexpr int32_t kMaxGridYZ = 65535;  // launch grid limit in y and z (one prompt per index)

}  // namespace

extern "C" {

TG_API int tg_abi_version(void) { return TG_ABI_VERSION; }

TG_API const char* tg_status_string(int status) {
  switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
    case TG_ERR_HIP: return "TG_ERR_HIP";
    case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE";
    default: return "TG_UNKNOWN_STATUS";
  }
}

TG_API const char* tg_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
static tg_status check_gate(const char* what, tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                            const void* h, int64_t ld_h, const void* w1, const float* w2, const float* g) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "%s: unknown dtype %d", what, (int)dtype);
  if (n < 0 || n > kMaxI32) return fail(TG_ERR_INVALID_ARG, "%s: n=%lld out of range", what, (long long)n);
  if (d <= 0 || hidden <= 0) return fail(TG_ERR_INVALID_ARG, "%s: d and hidden must be positive", what);
  if (ld_h < d) return fail(TG_ERR_INVALID_ARG, "%s: ld_h=%lld < d=%d", what, (long long)ld_h, d);
  const int es = elem_size(dtype);
  if ((ld_h * es) % 16 != 0) return fail(TG_ERR_INVALID_ARG, "%s: ld_h*elem_size must be a multiple of 16 bytes", what);
  if (dtype == TG_BF16) {
    if (d % 64 != 0) return fail(TG_ERR_UNSUPPORTED, "%s bf16: d=%d must be a multiple of 64", what, d);
    if (hidden != 64 && hidden != 128 && hidden != 256)
      return fail(TG_ERR_UNSUPPORTED, "%s bf16: hidden=%d must be 64, 128 or 256", what, hidden);
  } else {
    if (d % 4 != 0) return fail(TG_ERR_UNSUPPORTED, "%s fp32: d=%d must be a multiple of 4", what, d);
    if (hidden > 1024) return fail(TG_ERR_UNSUPPORTED, "%s fp32: hidden=%d > 1024", what, hidden);
  }
  if (n == 0) return TG_OK;
  if (!h || !w1 || !w2 || !g) return fail(TG_ERR_INVALID_ARG, "%s: NULL h, w1, w2 or g", what);
  if (!aligned16(h) || !aligned16(w1)) return fail(TG_ERR_INVALID_ARG, "%s: h and w1 must be 16-byte aligned", what);
  return TG_OK;
}

static hipError_t launch_gate(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden, const void* h, int64_t ld_h,
                              const void* w1, const float* b1, const float* w2, float b2, float* g, float* s,
                              hipStream_t stream) {
  if (dtype == TG_BF16) return tg::launch_gate_bf16(n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, stream);
  return tg::launch_gate_f32(n, d, hidden, static_cast<const float*>(h), ld_h, static_cast<const float*>(w1), b1,
                             w2, b2, g, s, stream);
}

TG_API tg_status tg_gate_score(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                               const void* h, int64_t ld_h, const void* w1, const float* b1,
                               const float* w2, float b2, float* g, float* s,
                               hipStream_t stream) {
  tg_status st = check_gate("gate", dtype, n, d, hidden, h, ld_h, w1, w2, g);
  if (st != TG_OK || n == 0) return st == TG_OK ? ok() : st;
  return from_hip(launch_gate(dtype, n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, stream), "gate");
}

static tg_status gate_select_impl(const char* what, tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                                  const void* h, int64_t ld_h, const void* w1, const float* b1, const float* w2,
                                  float b2, int64_t k, int64_t q_len, float* g, float* s, int32_t* idx, void* h_out,
                                  float* g_out, int32_t* pos_out, void* workspace, int64_t workspace_bytes,
                                  hipStream_t stream) {
  tg_status st = check_gate(what, dtype, n, d, hidden, h, ld_h, w1, w2, g);
  if (st != TG_OK) return st;
  if (k < 0) return fail(TG_ERR_INVALID_ARG, "%s: k=%lld < 0", what, (long long)k);
  const int64_t kept = k < n ? k : n;
  if (q_len < 0 || q_len > kept)
    return fail(TG_ERR_INVALID_ARG, "%s: q_len=%lld outside [0, min(k, n)=%lld]", what, (long long)q_len,
                (long long)kept);
  if (n == 0) return ok();
  if (!idx || !workspace) return fail(TG_ERR_INVALID_ARG, "%s: NULL idx or workspace", what);
  if (!aligned16(workspace)) return fail(TG_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
  const int64_t need = tg::select_mw_workspace_bytes(n);
  if (workspace_bytes < need)
    return fail(TG_ERR_WORKSPACE, "%s: workspace of %lld bytes, %lld needed", what, (long long)workspace_bytes,
                (long long)need);
  const bool gather = h_out != nullptr || g_out != nullptr || pos_out != nullptr;
  if (gather) {
    if (!h_out) return fail(TG_ERR_INVALID_ARG, "%s: NULL h_out", what);
    if (!aligned16(h_out)) return fail(TG_ERR_INVALID_ARG, "%s: h_out must be 16-byte aligned", what);
  }
  const int64_t doc = n - q_len, kd = kept - q_len;
  hipError_t e;
  if (dtype == TG_BF16 && kd > 0 && kd < doc && doc <= tg::gate_select_block_tokens(hidden)) {
    e = tg::launch_gate_select_bf16(n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, k, q_len, idx, workspace, h_out,
                                    g_out, pos_out, stream);
  } else {
    // fp32, a budget with nothing to rank, or a document longer than the
    // gate's last workgroup holds in LDS: the gate, then the selection
    // kernels (the one-workgroup kernel writes the identity or the tail
    // directly when kd says so; long documents take the multi-workgroup
    // form), then the gather.
    e = launch_gate(dtype, n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, stream);
    if (e == hipSuccess) e = tg::launch_select_mw(g, n, k, q_len, idx, workspace, true, stream);
    if (e == hipSuccess && gather)
      e = tg::launch_gather(elem_size(dtype), n, kept, d, idx, h, ld_h, g_out ? g : nullptr, h_out, g_out, pos_out,
                            nullptr, nullptr, 1, kept, stream);
  }
  return from_hip(e, what);
}

TG_API tg_status tg_gate_select(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden, const void* h, int64_t ld_h,
                                const void* w1, const float* b1, const float* w2, float b2, int64_t k,
                                int64_t q_len, float* g, float* s, int32_t* idx, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream) {
  return gate_select_impl("gate_select", dtype, n, d, hidden, h, ld_h, w1, b1, w2, b2, k, q_len, g, s, idx, nullptr,
                          nullptr, nullptr, workspace, workspace_bytes, stream);
}

TG_API tg_status tg_gate_select_gather(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden, const void* h,
                                       int64_t ld_h, const void* w1, const float* b1, const float* w2, float b2,
                                       int64_t k, int64_t q_len, float* g, float* s, int32_t* idx, void* h_out,
                                       float* g_out, int32_t* pos_out, void* workspace, int64_t workspace_bytes,
                                       hipStream_t stream) {
  if (!h_out) return fail(TG_ERR_INVALID_ARG, "gate_select_gather: NULL h_out");
  return gate_select_impl("gate_select_gather", dtype, n, d, hidden, h, ld_h, w1, b1, w2, b2, k, q_len, g, s, idx,
                          h_out, g_out, pos_out, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
TG_API tg_status tg_select_topk(const float* g, int64_t n, int64_t k, int64_t q_len,
                                int32_t* idx, hipStream_t stream) {
  if (n < 0 || n > kMaxI32) return fail(TG_ERR_INVALID_ARG, "select: n=%lld out of range", (long long)n);
  if (k < 0) return fail(TG_ERR_INVALID_ARG, "select: k=%lld < 0", (long long)k);
  const int64_t kept = k < n ? k : n;
  if (q_len < 0 || q_len > kept)
    return fail(TG_ERR_INVALID_ARG, "select: q_len=%lld outside [0, min(k, n)=%lld]", (long long)q_len,
                (long long)kept);
  if (n == 0) return ok();
  if (!g || !idx) return fail(TG_ERR_INVALID_ARG, "select: NULL g or idx");
  return from_hip(tg::launch_select(g, n, k, q_len, nullptr, nullptr, 1, n, idx, nullptr, stream),
                  "select");
}

TG_API int64_t tg_select_topk_workspace_size(int64_t n) {
  if (n < 0 || n > kMaxI32) return -1;
  return tg::select_mw_workspace_bytes(n);
}

TG_API tg_status tg_select_topk_ws(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx,
                                   void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n > kMaxI32) return fail(TG_ERR_INVALID_ARG, "select_ws: n=%lld out of range", (long long)n);
  if (k < 0) return fail(TG_ERR_INVALID_ARG, "select_ws: k=%lld < 0", (long long)k);
  const int64_t kept = k < n ? k : n;
  if (q_len < 0 || q_len > kept)
    return fail(TG_ERR_INVALID_ARG, "select_ws: q_len=%lld outside [0, min(k, n)=%lld]", (long long)q_len,
                (long long)kept);
  if (n == 0) return ok();
  if (!g || !idx || !workspace) return fail(TG_ERR_INVALID_ARG, "select_ws: NULL g, idx or workspace");
  if (!aligned16(workspace)) return fail(TG_ERR_INVALID_ARG, "select_ws: workspace must be 16-byte aligned");
  const int64_t need = tg::select_mw_workspace_bytes(n);
  if (workspace_bytes < need)
    return fail(TG_ERR_WORKSPACE, "select_ws: workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  return from_hip(tg::launch_select_mw(g, n, k, q_len, idx, workspace, false, stream), "select_ws");
}

TG_API tg_status tg_select_topk_varlen(const float* g, const int32_t* cu_seqlens,
                                       const int32_t* q_lens, int32_t batch, int64_t max_seqlen,
                                       int64_t k, int32_t* idx_local, int32_t* cu_kept,
                                       hipStream_t stream) {
  if (batch < 0) return fail(TG_ERR_INVALID_ARG, "select_varlen: batch < 0");
  if (max_seqlen < 0 || max_seqlen > kMaxI32) return fail(TG_ERR_INVALID_ARG, "select_varlen: max_seqlen out of range");
  if (k < 0) return fail(TG_ERR_INVALID_ARG, "select_varlen: k < 0");
  if (batch == 0) return ok();
  if (!g || !cu_seqlens || !q_lens || !idx_local || !cu_kept)
    return fail(TG_ERR_INVALID_ARG, "select_varlen: NULL pointer argument");
  return from_hip(tg::launch_select(g, 0, k, 0, cu_seqlens, q_lens, batch, max_seqlen, idx_local,
                                    cu_kept, stream),
                  "select_varlen");
}

// ---------------------------------------------------------------------------
static tg_status check_gather_common(tg_dtype dtype, int32_t d, const void* h, int64_t ld_h,
                                     const float* g, void* h_out, float* g_out) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "gather: unknown dtype %d", (int)dtype);
  const int es = elem_size(dtype);
  if (d <= 0) return fail(TG_ERR_INVALID_ARG, "gather: d must be positive");
  if ((int64_t)d * es % 16 != 0) return fail(TG_ERR_UNSUPPORTED, "gather: d*elem_size must be a multiple of 16 bytes");
  if (ld_h < d || (ld_h * es) % 16 != 0) return fail(TG_ERR_INVALID_ARG, "gather: ld_h must be >= d with 16-byte rows");
  if ((g == nullptr) != (g_out == nullptr)) return fail(TG_ERR_INVALID_ARG, "gather: pass both g and g_out, or neither");
  if (!h || !h_out) return fail(TG_ERR_INVALID_ARG, "gather: NULL h or h_out");
  if (!aligned16(h) || !aligned16(h_out)) return fail(TG_ERR_INVALID_ARG, "gather: h and h_out must be 16-byte aligned");
  return TG_OK;
}

TG_API tg_status tg_gather(tg_dtype dtype, int64_t n, int64_t n_kept, int32_t d, const int32_t* idx,
                           const void* h, int64_t ld_h, const float* g, void* h_out, float* g_out,
                           int32_t* pos_out, hipStream_t stream) {
  if (n < 0 || n > kMaxI32 || n_kept < 0 || n_kept > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "gather: n or n_kept out of range");
  if (n_kept == 0) return ok();
  tg_status st = check_gather_common(dtype, d, h, ld_h, g, h_out, g_out);
  if (st != TG_OK) return st;
  if (!idx) return fail(TG_ERR_INVALID_ARG, "gather: NULL idx");
  return from_hip(tg::launch_gather(elem_size(dtype), n, n_kept, d, idx, h, ld_h, g, h_out, g_out,
                                    pos_out, nullptr, nullptr, 1, n_kept, stream),
                  "gather");
}

TG_API tg_status tg_gather_varlen(tg_dtype dtype, const int32_t* cu_seqlens, const int32_t* cu_kept,
                                  int32_t batch, int64_t max_kept, int32_t d,
                                  const int32_t* idx_local, const void* h, int64_t ld_h,
                                  const float* g, void* h_out, float* g_out, int32_t* pos_out,
                                  hipStream_t stream) {
  if (batch < 0 || max_kept < 0 || max_kept > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "gather_varlen: batch or max_kept out of range");
  if (batch == 0 || max_kept == 0) return ok();
  if (batch > kMaxGridYZ) return fail(TG_ERR_UNSUPPORTED, "gather_varlen: batch above %d", kMaxGridYZ);
  tg_status st = check_gather_common(dtype, d, h, ld_h, g, h_out, g_out);
  if (st != TG_OK) return st;
  if (!idx_local || !cu_seqlens || !cu_kept) return fail(TG_ERR_INVALID_ARG, "gather_varlen: NULL pointer argument");
  return from_hip(tg::launch_gather(elem_size(dtype), 0, 0, d, idx_local, h, ld_h, g, h_out, g_out,
                                    pos_out, cu_seqlens, cu_kept, batch, max_kept, stream),
                  "gather_varlen");
}

// ---------------------------------------------------------------------------
TG_API tg_status tg_rope_table(float* cos_sin, int64_t max_pos, int32_t dh, double base,
                               hipStream_t stream) {
  if (max_pos < 0 || max_pos > kMaxI32) return fail(TG_ERR_INVALID_ARG, "rope_table: max_pos out of range");
  if (dh <= 0 || dh % 2 != 0 || dh > 256) return fail(TG_ERR_INVALID_ARG, "rope_table: dh must be even and <= 256");
  if (!(base > 1.0)) return fail(TG_ERR_INVALID_ARG, "rope_table: base must be > 1");
  if (max_pos == 0) return ok();
  if (!cos_sin) return fail(TG_ERR_INVALID_ARG, "rope_table: NULL cos_sin");
  return from_hip(tg::launch_rope_table(cos_sin, max_pos, dh, base, stream), "rope_table");
}

TG_API tg_status tg_rope_kv(tg_dtype dtype, int64_t n_kept, int32_t hq, int32_t hkv, int32_t dh,
                            const int32_t* pos, const float* cos_sin, int64_t max_pos, void* q,
                            const void* k, const void* v, void* k_cache, void* v_cache,
                            hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "rope_kv: unknown dtype %d", (int)dtype);
  if (n_kept < 0 || n_kept > kMaxI32 || max_pos < 0 || max_pos > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "rope_kv: n_kept or max_pos out of range");
  if (hq <= 0 || hkv <= 0) return fail(TG_ERR_INVALID_ARG, "rope_kv: head counts must be positive");
  if (dh <= 0 || dh % 16 != 0 || dh > 256) return fail(TG_ERR_UNSUPPORTED, "rope_kv: dh=%d must be a multiple of 16, <= 256", dh);
  if (n_kept == 0) return ok();
  if (!pos || !cos_sin || !q || !k || !v || !k_cache || !v_cache)
    return fail(TG_ERR_INVALID_ARG, "rope_kv: NULL pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(cos_sin))
    return fail(TG_ERR_INVALID_ARG, "rope_kv: tensors must be 16-byte aligned");
  return from_hip(tg::launch_rope_kv(elem_size(dtype), n_kept, hq, hkv, dh, pos, cos_sin, max_pos, q, k,
                                     v, k_cache, v_cache, stream),
                  "rope_kv");
}

// ---------------------------------------------------------------------------
static tg_status check_attn(tg_dtype dtype, int64_t max_rows, int32_t hq, int32_t hkv, int32_t dh,
                            float scale, const void* q, const void* k, const void* v, const float* g,
                            const int32_t* pos, void* o) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "attn: unknown dtype %d", (int)dtype);
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(TG_ERR_INVALID_ARG, "attn: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  if (dh != 64 && dh != 128) return fail(TG_ERR_UNSUPPORTED, "attn: dh=%d must be 64 or 128", dh);
  if (max_rows * hkv * dh * elem_size(dtype) >= (int64_t(1) << 31))
    return fail(TG_ERR_UNSUPPORTED, "attn: one prompt's K (or V) must be below 2 GiB");
  if (!(scale > 0.0f) || scale != scale) return fail(TG_ERR_INVALID_ARG, "attn: scale must be > 0");
  (void)g;  // NULL: no gate
  if (!q || !k || !v || !pos || !o) return fail(TG_ERR_INVALID_ARG, "attn: NULL pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(TG_ERR_INVALID_ARG, "attn: q, k, v and o must be 16-byte aligned");
  return TG_OK;
}

static hipError_t dispatch_attn(tg_dtype dtype, int64_t total, const int32_t* cu, int batch,
                                int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh, float scale,
                                const void* q, const void* k, const void* v, const float* g,
                                const float* head_gain, const int32_t* pos, void* o, float* lse,
                                hipStream_t stream) {
  if (dtype == TG_BF16)
    return tg::launch_attn_bf16(total, cu, batch, max_seqlen, hq, hkv, dh, scale, q, k, v, g, head_gain,
                                pos, o, lse, stream);
  return tg::launch_attn_f32(total, cu, batch, max_seqlen, hq, hkv, dh, scale,
                             static_cast<const float*>(q), static_cast<const float*>(k),
                             static_cast<const float*>(v), g, head_gain, static_cast<float*>(o),
                             lse, stream);
}

TG_API tg_status tg_gated_attn(tg_dtype dtype, int64_t n_kept, int32_t hq, int32_t hkv, int32_t dh,
                               float scale, const void* q, const void* k, const void* v,
                               const float* g, const int32_t* pos, void* o, float* lse,
                               hipStream_t stream) {
  if (n_kept < 0 || n_kept > kMaxI32) return fail(TG_ERR_INVALID_ARG, "attn: n_kept out of range");
  if (n_kept == 0) return ok();
  tg_status st = check_attn(dtype, n_kept, hq, hkv, dh, scale, q, k, v, g, pos, o);
  if (st != TG_OK) return st;
  return from_hip(dispatch_attn(dtype, n_kept, nullptr, 1, n_kept, hq, hkv, dh, scale, q, k, v, g, nullptr,
                                pos, o, lse, stream),
                  "attn");
}

TG_API tg_status tg_gated_attn_varlen(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                      int64_t max_seqlen, int64_t total, int32_t hq, int32_t hkv,
                                      int32_t dh, float scale, const void* q, const void* k,
                                      const void* v, const float* g, const int32_t* pos, void* o,
                                      float* lse, hipStream_t stream) {
  if (batch < 0 || max_seqlen < 0 || max_seqlen > kMaxI32 || total < 0 || total > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "attn_varlen: batch, max_seqlen or total out of range");
  if (batch == 0 || total == 0 || max_seqlen == 0) return ok();
  if (batch > kMaxGridYZ) return fail(TG_ERR_UNSUPPORTED, "attn_varlen: batch above %d", kMaxGridYZ);
  tg_status st = check_attn(dtype, max_seqlen, hq, hkv, dh, scale, q, k, v, g, pos, o);
  if (st != TG_OK) return st;
  if (!cu_seqlens) return fail(TG_ERR_INVALID_ARG, "attn_varlen: NULL cu_seqlens");
  return from_hip(dispatch_attn(dtype, total, cu_seqlens, batch, max_seqlen, hq, hkv, dh, scale, q, k, v,
                                g, nullptr, pos, o, lse, stream),
                  "attn_varlen");
}

TG_API tg_status tg_gated_attn_ex(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                  int64_t max_seqlen, int64_t total, int32_t hq, int32_t hkv,
                                  int32_t dh, float scale, const void* q, const void* k,
                                  const void* v, const float* g, const float* head_gain,
                                  const int32_t* pos, void* o, float* lse, hipStream_t stream) {
  if (total < 0 || total > kMaxI32) return fail(TG_ERR_INVALID_ARG, "attn_ex: total out of range");
  if (cu_seqlens) {
    if (batch < 0 || max_seqlen < 0 || max_seqlen > kMaxI32)
      return fail(TG_ERR_INVALID_ARG, "attn_ex: batch or max_seqlen out of range");
    if (batch == 0 || total == 0 || max_seqlen == 0) return ok();
    if (batch > kMaxGridYZ) return fail(TG_ERR_UNSUPPORTED, "attn_ex: batch above %d", kMaxGridYZ);
  } else {
    batch = 1;
    max_seqlen = total;
    if (total == 0) return ok();
  }
  tg_status st = check_attn(dtype, max_seqlen, hq, hkv, dh, scale, q, k, v, g, pos, o);
  if (st != TG_OK) return st;
  return from_hip(dispatch_attn(dtype, total, cu_seqlens, batch, max_seqlen, hq, hkv, dh, scale, q, k, v,
                                g, head_gain, pos, o, lse, stream),
                  "attn_ex");
}

// ---------------------------------------------------------------------------
static int64_t decode_ws_bytes(int32_t batch, int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh) {
  if (batch < 0 || max_seqlen < 0 || max_seqlen > kMaxI32 || hq <= 0 || hkv <= 0 || hq % hkv != 0 ||
      (dh != 64 && dh != 128))
    return -1;
  const int split = tg::decode_split_keys(batch, hkv, max_seqlen);
  int64_t nsplit = (max_seqlen + split - 1) / split;
  if (nsplit < 1) nsplit = 1;
  return (int64_t)batch * hq * nsplit * (dh + 2) * (int64_t)sizeof(float);
}

TG_API int64_t tg_decode_attn_workspace_size(int32_t batch, int64_t max_seqlen, int32_t hq, int32_t hkv,
                                             int32_t dh) {
  return decode_ws_bytes(batch, max_seqlen, hq, hkv, dh);
}

static tg_status check_decode(const char* what, tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                              int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh, float scale, const void* q,
                              const void* k_cache, const void* v_cache, void* o) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "%s: unknown dtype %d", what, (int)dtype);
  if (batch < 0 || max_seqlen < 0 || max_seqlen > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "%s: batch or max_seqlen out of range", what);
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(TG_ERR_INVALID_ARG, "%s: hq=%d must be a positive multiple of hkv=%d", what, hq, hkv);
  const int group = hq / hkv;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(TG_ERR_UNSUPPORTED, "%s: hq/hkv=%d must be 1, 2, 4 or 8", what, group);
  if (dh != 64 && dh != 128) return fail(TG_ERR_UNSUPPORTED, "%s: dh=%d must be 64 or 128", what, dh);
  if (!(scale > 0.0f) || scale != scale) return fail(TG_ERR_INVALID_ARG, "%s: scale must be > 0", what);
  if (batch == 0) return TG_OK;
  if (batch > kMaxGridYZ) return fail(TG_ERR_UNSUPPORTED, "%s: batch above %d", what, kMaxGridYZ);
  if (!cu_seqlens || !q || !k_cache || !v_cache || !o) return fail(TG_ERR_INVALID_ARG, "%s: NULL pointer argument", what);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(TG_ERR_INVALID_ARG, "%s: q, k_cache and v_cache must be 16-byte aligned", what);
  return TG_OK;
}

TG_API int64_t tg_decode_attn_noalloc_max_bytes(void) { return tg::kDecodeStaticScratchBytes; }

TG_API tg_status tg_decode_attn_noalloc(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                        int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh, float scale,
                                        const void* q, const void* k_cache, const void* v_cache, const float* g,
                                        const float* head_gain, void* o, float* lse, hipStream_t stream) {
  tg_status st = check_decode("decode_noalloc", dtype, cu_seqlens, batch, max_seqlen, hq, hkv, dh, scale, q, k_cache,
                              v_cache, o);
  if (st != TG_OK) return st;
  if (batch == 0) return ok();
  const int64_t need = decode_ws_bytes(batch, max_seqlen, hq, hkv, dh);
  if (need > tg::kDecodeStaticScratchBytes)
    return fail(TG_ERR_WORKSPACE, "decode_noalloc: needs %lld bytes of scratch, the static scratch holds %lld; "
                "use tg_decode_attn with a caller workspace", (long long)need,
                (long long)tg::kDecodeStaticScratchBytes);
  void* ws = nullptr;
  hipError_t e = tg::decode_static_scratch(&ws);
  if (e != hipSuccess) return from_hip(e, "decode_noalloc: looking up the static scratch");
  return from_hip(tg::launch_decode(elem_size(dtype), cu_seqlens, batch, max_seqlen, hq, hkv, dh, scale, q, k_cache,
                                    v_cache, g, head_gain, o, lse, static_cast<float*>(ws), stream),
                  "decode_noalloc");
}

TG_API tg_status tg_decode_attn(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh, float scale,
                                const void* q, const void* k_cache, const void* v_cache, const float* g,
                                const float* head_gain, void* o, float* lse, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "decode: unknown dtype %d", (int)dtype);
  if (batch < 0 || max_seqlen < 0 || max_seqlen > kMaxI32)
    return fail(TG_ERR_INVALID_ARG, "decode: batch or max_seqlen out of range");
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(TG_ERR_INVALID_ARG, "decode: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  const int group = hq / hkv;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(TG_ERR_UNSUPPORTED, "decode: hq/hkv=%d must be 1, 2, 4 or 8", group);
  if (dh != 64 && dh != 128) return fail(TG_ERR_UNSUPPORTED, "decode: dh=%d must be 64 or 128", dh);
  if (!(scale > 0.0f) || scale != scale) return fail(TG_ERR_INVALID_ARG, "decode: scale must be > 0");
  if (batch == 0) return ok();
  if (batch > kMaxGridYZ) return fail(TG_ERR_UNSUPPORTED, "decode: batch above %d", kMaxGridYZ);
  if (!cu_seqlens || !q || !k_cache || !v_cache || !o || !workspace)
    return fail(TG_ERR_INVALID_ARG, "decode: NULL pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
    return fail(TG_ERR_INVALID_ARG, "decode: q, k_cache, v_cache and workspace must be 16-byte aligned");
  const int64_t need = decode_ws_bytes(batch, max_seqlen, hq, hkv, dh);
  if (workspace_bytes < need)
    return fail(TG_ERR_WORKSPACE, "decode: workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)need);
  return from_hip(tg::launch_decode(elem_size(dtype), cu_seqlens, batch, max_seqlen, hq, hkv, dh, scale, q,
                                    k_cache, v_cache, g, head_gain, o, lse, static_cast<float*>(workspace),
                                    stream),
                  "decode");
}

// ---------------------------------------------------------------------------
static tg_status check_dense(const char* what, tg_dtype dtype, int64_t m, int64_t n, int64_t k, int n_mult,
                             const void* x, int64_t ld_x, const void* w, int64_t ld_w, void* y, int64_t ld_y) {
  if (!valid_dtype(dtype)) return fail(TG_ERR_INVALID_ARG, "%s: unknown dtype %d", what, (int)dtype);
  if (dtype != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "%s: only TG_BF16 is implemented", what);
  if (m < 0 || m > kMaxI32 - 256 || n <= 0 || k <= 0)
    return fail(TG_ERR_INVALID_ARG, "%s: m=%lld, n=%lld, k=%lld out of range", what, (long long)m, (long long)n,
                (long long)k);
  if (n % n_mult != 0 || k % 32 != 0)
    return fail(TG_ERR_UNSUPPORTED, "%s: n=%lld must be a multiple of %d and k=%lld of 32", what, (long long)n,
                n_mult, (long long)k);
  if (ld_x < k || ld_w < k || ld_y < n || ld_x % 8 != 0 || ld_w % 8 != 0)
    return fail(TG_ERR_INVALID_ARG, "%s: leading dimensions too small or not multiples of 8", what);
  if (((m + 127) / 128) * (n / 128) > kMaxI32)
    return fail(TG_ERR_UNSUPPORTED, "%s: product too large for one launch", what);
  if (!x || !w || !y) return fail(TG_ERR_INVALID_ARG, "%s: NULL pointer argument", what);
  if (!aligned16(x) || !aligned16(w)) return fail(TG_ERR_INVALID_ARG, "%s: x and w must be 16-byte aligned", what);
  if ((reinterpret_cast<uintptr_t>(y) & 1u) != 0) return fail(TG_ERR_INVALID_ARG, "%s: y must be 2-byte aligned", what);
  return TG_OK;
}

TG_API tg_status tg_linear(tg_dtype dtype, int64_t m, int32_t n, int32_t k, const void* x, int64_t ld_x,
                           const void* w, int64_t ld_w, const void* residual, int64_t ld_r, void* y, int64_t ld_y,
                           hipStream_t stream) {
  tg_status st = check_dense("linear", dtype, m, n, k, 256, x, ld_x, w, ld_w, y, ld_y);
  if (st != TG_OK) return st;
  if (residual && (ld_r < n || (reinterpret_cast<uintptr_t>(residual) & 1u) != 0))
    return fail(TG_ERR_INVALID_ARG, "linear: residual needs ld_r >= n and 2-byte alignment");
  if (residual == y && ld_r != ld_y)
    return fail(TG_ERR_INVALID_ARG, "linear: an in-place residual (residual == y) needs ld_r == ld_y");
  if (m == 0) return ok();
  return from_hip(tg::launch_gemm_bf16(residual ? 1 : 0, m, n, k, x, ld_x, w, nullptr, ld_w, residual, ld_r, y,
                                       ld_y, stream),
                  "linear");
}

TG_API tg_status tg_swiglu(tg_dtype dtype, int64_t m, int32_t f, int32_t k, const void* x, int64_t ld_x,
                           const void* w_gate, const void* w_up, int64_t ld_w, void* y, int64_t ld_y,
                           hipStream_t stream) {
  tg_status st = check_dense("swiglu", dtype, m, f, k, 128, x, ld_x, w_gate, ld_w, y, ld_y);
  if (st != TG_OK) return st;
  if (!w_up || !aligned16(w_up)) return fail(TG_ERR_INVALID_ARG, "swiglu: w_up must be 16-byte aligned, not NULL");
  if (m == 0) return ok();
  return from_hip(
      tg::launch_gemm_bf16(2, m, f, k, x, ld_x, w_gate, w_up, ld_w, nullptr, 0, y, ld_y, stream), "swiglu");
}

TG_API tg_status tg_qkv_proj(tg_dtype dtype, int64_t m, int32_t hq, int32_t hkv, int32_t dh, int32_t k,
                             const void* x, int64_t ld_x, const void* w_qkv, int64_t ld_w, void* q, void* k_out,
                             void* v_out, hipStream_t stream) {
  if (hq <= 0 || hkv <= 0 || dh <= 0 || ((int64_t)hq * dh) % 256 != 0 || ((int64_t)hkv * dh) % 256 != 0)
    return fail(TG_ERR_UNSUPPORTED, "qkv_proj: hq*dh and hkv*dh must be positive multiples of 256");
  const int64_t nq = (int64_t)hq * dh, nkv = (int64_t)hkv * dh, n = nq + 2 * nkv;
  if (n > kMaxI32) return fail(TG_ERR_INVALID_ARG, "qkv_proj: too many output columns");
  tg_status st = check_dense("qkv_proj", dtype, m, n, k, 256, x, ld_x, w_qkv, ld_w, q, n);
  if (st != TG_OK) return st;
  if (!k_out || !v_out || (reinterpret_cast<uintptr_t>(k_out) & 1u) || (reinterpret_cast<uintptr_t>(v_out) & 1u))
    return fail(TG_ERR_INVALID_ARG, "qkv_proj: k_out and v_out must be 2-byte aligned, not NULL");
  if (m == 0) return ok();
  return from_hip(tg::launch_gemm_bf16_split(0, m, n, k, x, ld_x, w_qkv, nullptr, ld_w, nullptr, 0, q, nq, k_out,
                                             nkv, nq, v_out, nkv, nq + nkv, stream),
                  "qkv_proj");
}

TG_API tg_status tg_check_positions(const int32_t* pos, int64_t total, const int32_t* cu_seqlens, int32_t batch,
                                    int32_t* first_bad, hipStream_t stream) {
  if (total < 0 || total > kMaxI32) return fail(TG_ERR_INVALID_ARG, "check_positions: total out of range");
  if (!first_bad) return fail(TG_ERR_INVALID_ARG, "check_positions: NULL first_bad");
  if (total > 0 && !pos) return fail(TG_ERR_INVALID_ARG, "check_positions: NULL pos");
  if (cu_seqlens && batch < 0) return fail(TG_ERR_INVALID_ARG, "check_positions: negative batch");
  return from_hip(tg::launch_check_positions(pos, total, cu_seqlens, cu_seqlens ? batch : 0, first_bad, stream),
                  "check_positions");
}

}  // extern "C"
