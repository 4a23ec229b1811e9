/*
 * tokengate.h -- C ABI of libtokengate.so, the MI355X (gfx950) hot path of
 * TokenGate's gated prefill.
 *
 * Sources, cited by page title and section only:
 *   [paper]  "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill
 *            with Learned Token Pruning" (paper page on thelatestinai.com),
 *            Abstract, Figure 1 (a)-(c) and the training-setup table (base
 *            model and LoRA configuration).
 *   [aitu]   The aitualizate.com news article on TokenGate, sections
 *            "2. Una red MLP aprende qué tokens conservar", "3. Las capas
 *            superiores procesan únicamente los tokens seleccionados",
 *            "Cómo consigue entrenar una selección top-K" and "Cómo identifica
 *            el contenido que puede podarse".
 *
 * The path, per prompt:  gate score (all N tokens) -> top-K select (question
 * tail always kept) -> gather of the kept rows, gate values and positions ->
 * per upper layer: RoPE + compact KV cache, then token-gated causal GQA
 * attention over the K kept tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer unless its comment says otherwise.  The
 *    caller allocates and owns every buffer; the library never allocates and
 *    keeps no state besides a thread-local error message (and the static
 *    scratch array of tg_decode_attn_noalloc).
 *  - Every call only enqueues work on `stream` (0 = the null stream) and returns
 *    without synchronising.  Calls are thread-safe; calls on different streams
 *    may run concurrently if their output buffers do not overlap.
 *  - Arguments are validated on the host before any HIP call.  A failed check
 *    returns TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED or TG_ERR_WORKSPACE,
 *    enqueues nothing and sets the message returned by tg_last_error().  A launch failure reported by HIP
 *    returns TG_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *    synchronisation.
 *  - n == 0 (nothing to do) returns TG_OK and enqueues nothing.
 *  - Dense tensors are contiguous and row-major in the shapes given; bf16 is
 *    IEEE bfloat16 stored in 2 bytes; every fp32 -> bf16 conversion rounds to
 *    nearest even.  Tensor pointers must be 16-byte aligned.
 *  - Gate values g are fp32.  Indices and positions are int32.
 *  - A packed ragged batch (cu_seqlens) holds at most 65535 prompts per call
 *    (one launch-grid row per prompt); larger batches give TG_ERR_UNSUPPORTED.
 *  - A call whose launch grid would exceed what one dispatch can count (2^32
 *    work-items in x, 65535 workgroups in y and z) returns TG_ERR_UNSUPPORTED
 *    before any HIP call: for example a gather or rope_kv over 2^26 or 2^24
 *    rows, or a select over 2^22 prompts.  Split such work over several calls.
 *  - Later rows beside the prefill path: decode attention over the compact
 *    cache (tg_decode_attn, which takes a caller workspace, as does the
 *    multi-workgroup select tg_select_topk_ws), the
 *    upper layers' dense products (tg_qkv_proj, tg_linear, tg_swiglu) and a
 *    device-side check of the position order (tg_check_positions).
 */
#ifndef TOKENGATE_H_
#define TOKENGATE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_API __attribute__((visibility("default")))

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, inconsistent sizes */
  TG_ERR_UNSUPPORTED = 2, /* valid request that this build has no kernel for */
  TG_ERR_WORKSPACE = 3,   /* caller workspace smaller than its size function asks for */
  TG_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} tg_status;

typedef enum tg_dtype {
  TG_FP32 = 0,
  TG_BF16 = 1
} tg_dtype;

/* Version of this ABI; bumped on any incompatible change. */
#define TG_ABI_VERSION 1
TG_API int tg_abi_version(void);

/* Static text for a status code ("TG_OK", ...). Never NULL. */
TG_API const char* tg_status_string(int status);

/* Detail of the last failing call made on this thread ("" if none). The
 * pointer stays valid until the next call on this thread. */
TG_API const char* tg_last_error(void);

/* ---------------------------------------------------------------------------
 * Stage 1 -- gate MLP.  [paper] Figure 1(b): a small scoring network scores
 * every hidden state; [aitu] section 2: the network reads each token's
 * post-attention residual state at the selection layer L.  This library's
 * reading of the network:
 *     a = W1 h_j + b1  (d -> hidden),  z = SiLU(a) = a * sigmoid(a),
 *     s_j = w2 . z + b2,               g_j = sigmoid(s_j)  in (0, 1).
 *
 *   dtype   TG_BF16: h and w1 are bf16, products accumulate in fp32 (MFMA) and
 *           the epilogue (bias, SiLU, w2 dot, sigmoid) runs in fp32.
 *           TG_FP32: h and w1 are fp32, all arithmetic fp32.
 *   n       tokens (rows of h), >= 0.
 *   d       hidden size.  bf16: multiple of 64.  fp32: multiple of 4.
 *   hidden  gate MLP width.  bf16: 64, 128 or 256.  fp32: 1..1024.
 *   h       [n, ld_h] rows; only the first d columns are read.  ld_h >= d, and
 *           ld_h * element size must be a multiple of 16 bytes.
 *   w1      [hidden, d] (nn.Linear layout: row k is unit k's input weights).
 *   b1      [hidden] fp32, or NULL for zero.
 *   w2      [hidden] fp32.
 *   b2      output bias.
 *   g       [n] fp32 output: gate values.
 *   s       [n] fp32 output: scores (pre-sigmoid), or NULL.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_gate_score(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                               const void* h, int64_t ld_h, const void* w1,
                               const float* b1, const float* w2, float b2,
                               float* g, float* s, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Stage 2 -- top-K selection.  [paper] Figure 1(a),(b): a top-K selector at
 * layer L keeps K of the N tokens; [aitu] sections 3 and "Cómo identifica el
 * contenido que puede podarse": only the document may be pruned, the question
 * is never removed, and the budget is the maximum number of kept tokens.
 * This library's reading (exact, one correct answer):
 *   - K counts every kept token, question included: kept = min(k, n), of which
 *     the q_len trailing tokens [n - q_len, n) are always kept and
 *     kd = min(k, n) - q_len are chosen among the document [0, n - q_len).
 *   - Document tokens are ranked by g as fp32 numbers, larger first, ties to
 *     the lower index; -0 equals +0; NaN ranks below every number.
 *   - idx receives the kept indices in ascending order (the tail last).
 *   - k >= n keeps every token (idx = 0..n-1).
 *
 *   g      [n] fp32 gate values.
 *   n      tokens, 0 <= n < 2^31.
 *   k      budget, >= q_len.      q_len  0 <= q_len <= min(k, n).
 *   idx    [min(k, n)] int32 output.
 * Errors: q_len > min(k, n), negative sizes, NULL pointers -> INVALID_ARG.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_select_topk(const float* g, int64_t n, int64_t k, int64_t q_len,
                                int32_t* idx, hipStream_t stream);

/* The same selection (same arguments, same output, bit for bit) in three
 * short kernels: a clear of the workspace's counts; ceil((n - q_len) / 4096)
 * workgroups that count the top 11 bits of their keys, the last of which to
 * finish (an arrival counter in the workspace, no waiting) ranks alone; and
 * one workgroup per 64 tokens that writes the kept indices.  It takes a
 * caller workspace of at least tg_select_topk_workspace_size(n) bytes
 * (4 (R64(2112 + 3 ceil(n / 64) + ceil(n / 8)) + R256(n)), where Rm rounds up
 * to a multiple of m: about 4.4 n + 8.5 KB), 16-byte aligned, whose contents
 * need not be initialised.  Calls that share a workspace must be ordered on one stream.
 * Documents (n - q_len) longer than 32768 tokens, which one workgroup would
 * have to re-read block by block in every pass, run six short kernels over
 * 2048-key chunks instead (a clear, three histogram passes, the per-chunk
 * counts, the writes of idx), with no workgroup waiting for another;
 * documents longer than 2^24 tokens, budgets that keep the whole document and
 * budgets that keep none of it run the one-workgroup kernel of
 * tg_select_topk.  The multi-workgroup forms leave the workspace's first
 * 8196 bytes zero, as tg_gate_select expects; the one-workgroup kernel does
 * not touch the workspace.
 * Errors: as tg_select_topk; a NULL or misaligned workspace -> INVALID_ARG;
 * a workspace smaller than tg_select_topk_workspace_size(n) -> WORKSPACE. */
TG_API int64_t tg_select_topk_workspace_size(int64_t n); /* -1 for n outside [0, 2^31) */
TG_API tg_status tg_select_topk_ws(const float* g, int64_t n, int64_t k, int64_t q_len,
                                   int32_t* idx, void* workspace, int64_t workspace_bytes,
                                   hipStream_t stream);

/* Stages 1 and 2 in two kernels: tg_gate_score over the n tokens, then
 * tg_select_topk over the scores it wrote.  [paper] Figure 1(b): the selector
 * ranks the importance scores of the gate module at layer L.  Each
 * workgroup of the gate counts the top 11 bits of its document scores into
 * the workspace; the last workgroup to finish ranks every score (the kd-th
 * largest key, how many keys equal to it are kept, and the counts before
 * every 64-token chunk); a second kernel, one workgroup per 64 tokens, writes
 * idx.  The outputs equal those of tg_gate_score followed by tg_select_topk
 * on the g this call writes (bit for bit for idx).
 *
 *   Arguments as tg_gate_score, plus k, q_len, idx as tg_select_topk.
 *   workspace  at least tg_select_topk_workspace_size(n) bytes, 16-byte
 *              aligned, ZERO-FILLED before its first use (e.g. allocated
 *              zeroed).  Every call leaves its counts and arrival counter
 *              (the first 8196 bytes) zero again, so a caller reuses it
 *              across calls with no clearing.  Counts that do not add up make
 *              the call count the keys again (slower, same result); a non-zero
 *              counter on entry (memory that is neither fresh zeros nor left by
 *              a previous call) gives undefined indices, never an access
 *              outside the arguments.  Calls sharing a workspace must be
 *              ordered on one stream.
 *   dtype      TG_BF16 runs the fused kernels while the document
 *              (n - q_len) fits what the gate's last workgroup holds in LDS
 *              (32768 tokens at hidden 256, 24576 at 128, 18432 at 64);
 *              longer documents, and TG_FP32, run the gate followed by
 *              tg_select_topk_ws on the same workspace (same results).
 * Errors: those of tg_gate_score and tg_select_topk_ws.
 */
TG_API tg_status tg_gate_select(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                                const void* h, int64_t ld_h, const void* w1, const float* b1,
                                const float* w2, float b2, int64_t k, int64_t q_len,
                                float* g, float* s, int32_t* idx, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream);

/* Stages 1 to 3 in two kernels: tg_gate_select, with the kernel that places
 * the kept tokens also copying them: h_out[i] = h[idx[i]], g_out[i] =
 * g[idx[i]], pos_out[i] = idx[i] (tg_gather's outputs, bit for bit).  The
 * ranking lists the kept tokens as items of at most 8 rows (a 64-token
 * chunk with many kept tokens gives several items), one workgroup each, so
 * the copy stays balanced however the kept tokens cluster.
 * [paper] Figure 1(b): the selector forwards the kept hidden states together
 * with their importance scores.
 *   h_out    [min(k, n), d] contiguous, 16-byte aligned (not NULL).
 *   g_out    [min(k, n)] fp32, or NULL.   pos_out [min(k, n)] int32, or NULL.
 * Other arguments, workspace rules and errors as tg_gate_select. */
TG_API tg_status tg_gate_select_gather(tg_dtype dtype, int64_t n, int32_t d, int32_t hidden,
                                       const void* h, int64_t ld_h, const void* w1,
                                       const float* b1, const float* w2, float b2, int64_t k,
                                       int64_t q_len, float* g, float* s, int32_t* idx,
                                       void* h_out, float* g_out, int32_t* pos_out,
                                       void* workspace, int64_t workspace_bytes,
                                       hipStream_t stream);

/* Ragged batch of prompts packed along the token axis.
 *   g           [total] fp32, prompt b occupies [cu_seqlens[b], cu_seqlens[b+1]).
 *   cu_seqlens  [batch + 1] int32 (device), non-decreasing, cu_seqlens[0] = 0.
 *   q_lens      [batch] int32 (device); 0 <= q_lens[b] <= min(k, N_b).
 *   batch       number of prompts, >= 0.
 *   max_seqlen  host-side upper bound of every N_b (chooses the kernel).
 *   k           per-prompt budget.
 *   idx_local   [sum_b min(k, N_b)] int32 output: prompt b's kept positions,
 *               relative to its start, at offset cu_kept[b].
 *   cu_kept     [batch + 1] int32 output: offsets of each prompt's kept tokens.
 * max_seqlen only chooses the kernel's register footprint: a prompt longer
 * than it is still ranked exactly (its keys are re-read once per radix pass).
 * A prompt whose q_len is outside [0, min(k, N_b)] gets -1 in every one of
 * its idx_local entries; the other prompts are unaffected. */
TG_API tg_status tg_select_topk_varlen(const float* g, const int32_t* cu_seqlens,
                                       const int32_t* q_lens, int32_t batch,
                                       int64_t max_seqlen, int64_t k, int32_t* idx_local,
                                       int32_t* cu_kept, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Stage 3 -- gather.  [paper] Figure 1(b): the selector forwards the kept
 * hidden states together with their importance scores; [aitu] section 3:
 * the layers above L receive only the kept tokens.  Each kept token also
 * carries its original position (its index in the prompt).
 *   h_out[i] = h[idx[i]],  g_out[i] = g[idx[i]],  pos_out[i] = idx[i].
 *
 *   n          rows of h (idx entries must lie in [0, n)).
 *   n_kept     entries of idx.
 *   d          row length in elements; d * element size multiple of 16 bytes.
 *   h          [n, ld_h]; h_out [n_kept, d] contiguous.
 *   g, g_out   fp32, or both NULL to skip.   pos_out int32 [n_kept] or NULL.
 * An idx entry outside [0, n) yields a zero row, g_out = 0 and pos_out = -1.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_gather(tg_dtype dtype, int64_t n, int64_t n_kept, int32_t d,
                           const int32_t* idx, const void* h, int64_t ld_h,
                           const float* g, void* h_out, float* g_out, int32_t* pos_out,
                           hipStream_t stream);

/* Packed-batch gather: prompt b's kept rows are h[cu_seqlens[b] + idx_local[i]]
 * for i in [cu_kept[b], cu_kept[b+1]); pos_out = idx_local (positions within
 * the prompt).  max_kept bounds every prompt's kept count (host side).  An
 * entry outside its prompt yields a zero row, g_out = 0 and pos_out = -1. */
TG_API tg_status tg_gather_varlen(tg_dtype dtype, const int32_t* cu_seqlens,
                                  const int32_t* cu_kept, int32_t batch, int64_t max_kept,
                                  int32_t d, const int32_t* idx_local, const void* h,
                                  int64_t ld_h, const float* g, void* h_out, float* g_out,
                                  int32_t* pos_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Stage 5 -- RoPE at original positions and a KV cache for kept tokens only.
 * [aitu] section 3: discarded tokens create no key/value cache entries in the
 * layers above L.  Position encoding is not on the pages; this library uses
 * the rotate-half form (pairs (i, i + dh/2)) with angle pos * base^(-2i/dh).
 *
 * tg_rope_table fills cos_sin [max_pos, dh] fp32: row p holds
 * cos(p*theta_0..theta_{dh/2-1}) then sin(...), computed in fp64 on the device.
 *
 * tg_rope_kv, per kept token i at position pos[i]:
 *   q[i]        rotated in place             q [n_kept, hq, dh]
 *   k_cache[i]  = rotated k[i]               k, k_cache [n_kept, hkv, dh]
 *   v_cache[i]  = v[i]  (copy; skipped when v_cache == v)
 * dh: a multiple of 16, at most 256.  A position outside [0, max_pos) gives
 * zero outputs for that token.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_rope_table(float* cos_sin, int64_t max_pos, int32_t dh, double base,
                               hipStream_t stream);

TG_API tg_status tg_rope_kv(tg_dtype dtype, int64_t n_kept, int32_t hq, int32_t hkv,
                            int32_t dh, const int32_t* pos, const float* cos_sin,
                            int64_t max_pos, void* q, const void* k, const void* v,
                            void* k_cache, void* v_cache, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Stage 4 -- token-gated causal GQA attention over the kept tokens.
 * [paper] Figure 1(c): each attention weight is multiplied by its key's gate
 * value g_j (the weights are then renormalised); [paper] Abstract and [aitu]
 * "Cómo consigue entrenar una selección top-K": the importance score acts as a
 * bias on the attention logits.  Computed form, for query head h (KV head
 * h / (hq/hkv)) and kept query i:
 *   o_i = sum_{j: pos_j <= pos_i} softmax_j(scale * q_i.k_j + ln max(g_j, FLT_MIN)) v_j
 *   lse_i = ln sum_{j: pos_j <= pos_i} exp(scale * q_i.k_j + ln max(g_j, FLT_MIN))
 * Gain 1 and temperature 1 (the pages' raw-bias form).
 *
 *   dtype   TG_BF16: bf16 q/k/v/o, MFMA products with fp32 accumulation and an
 *           fp32 softmax.  TG_FP32: fp32 throughout.
 *   n_kept  kept tokens (rows of q, k, v).
 *   hq,hkv  heads; hq % hkv == 0.     dh: 64 or 128.
 *   scale   logit scale (1/sqrt(dh) for the standard form); must be > 0.
 *   q       [n_kept, hq, dh] (rotated); k, v [n_kept, hkv, dh] (the cache).
 *   g       [n_kept] fp32 gate values of the kept tokens, or NULL for no gate
 *           (every key weighs 1: plain causal GQA attention, the form of the
 *           full-context layers at or below the selection layer).
 *   pos     [n_kept] int32 original positions, strictly increasing (the
 *           order select + gather produce).  Precondition, not checked:
 *           both dtypes apply the causal mask by kept index (key j visible
 *           to query i iff j <= i), which is the mask above whenever the
 *           positions strictly increase; the values of pos are not read
 *           (tg_check_positions verifies the precondition on the device).
 *           Must be non-NULL.
 *   o       [n_kept, hq, dh] output, dtype.
 *   lse     [hq, n_kept] fp32 output (natural log), or NULL.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_gated_attn(tg_dtype dtype, int64_t n_kept, int32_t hq, int32_t hkv,
                               int32_t dh, float scale, const void* q, const void* k,
                               const void* v, const float* g, const int32_t* pos, void* o,
                               float* lse, hipStream_t stream);

/* Packed ragged batch: prompt b owns rows [cu_seqlens[b], cu_seqlens[b+1]) of
 * q, k, v, g, pos, o, and columns of lse [hq, total]; prompts never attend to
 * each other.  max_seqlen (host) bounds every prompt's row count; total is
 * the number of packed rows.  pos holds positions within each prompt. */
TG_API tg_status tg_gated_attn_varlen(tg_dtype dtype, const int32_t* cu_seqlens,
                                      int32_t batch, int64_t max_seqlen, int64_t total,
                                      int32_t hq, int32_t hkv, int32_t dh, float scale,
                                      const void* q, const void* k, const void* v,
                                      const float* g, const int32_t* pos, void* o,
                                      float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Gated attention with a per-head gain on the gate bias.  [paper] Abstract
 * and the page's discussion of the bias: each head scales the importance
 * bias with its own gain and a temperature, whose exact forms the pages do not
 * print.  This library's reading: head h uses the bias
 *     gamma_h * ln max(g_j, FLT_MIN),     gamma_h = head_gain[h]
 * (gain over temperature, any finite value; gamma_h = 0 switches the gate off
 * for that head, gamma_h = 1 is tg_gated_attn).
 *
 *   cu_seqlens  [batch + 1] int32 (device) for a packed ragged batch, as in
 *               tg_gated_attn_varlen; or NULL for one prompt of `total` rows
 *               (batch and max_seqlen are then ignored).
 *   g           [total] fp32, or NULL for no gate.
 *   head_gain   [hq] fp32 (device), or NULL for gamma_h = 1.
 *   Other arguments and errors as tg_gated_attn_varlen.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_gated_attn_ex(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                  int64_t max_seqlen, int64_t total, int32_t hq, int32_t hkv,
                                  int32_t dh, float scale, const void* q, const void* k,
                                  const void* v, const float* g, const float* head_gain,
                                  const int32_t* pos, void* o, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode attention over the compact KV cache.  [aitu] section 3: past the
 * selection layer only the kept tokens have keys and values, so each newly
 * generated token attends over its sequence's compact cache.  Decode itself
 * is not described on the pages; this library's reading: the kept prompt
 * keys keep their gate bias, tokens appended while generating carry g = 1
 * (bias 0), and every cached key precedes the new token (no mask).  For
 * sequence b and query head h (KV head h / (hq/hkv)):
 *   o[b,h]   = sum_j softmax_j(scale * q[b,h].k_j + gamma_h ln max(g_j, FLT_MIN)) v_j
 *   lse[b,h] = ln sum_j exp(scale * q[b,h].k_j + gamma_h ln max(g_j, FLT_MIN))
 * over j in [cu_seqlens[b], cu_seqlens[b+1]).  An empty cache gives o = 0
 * and lse = -inf.
 *
 *   dtype       TG_BF16: bf16 q/caches/o, fp32 products and softmax.
 *               TG_FP32: fp32 throughout.
 *   cu_seqlens  [batch + 1] int32 (device), non-decreasing, cu_seqlens[0] = 0;
 *               cache lengths must not exceed max_seqlen (host).  Not checked.
 *   hq, hkv     heads; hq / hkv in {1, 2, 4, 8}.   dh: 64 or 128.
 *   scale       logit scale, > 0.
 *   q           [batch, hq, dh] (rotated) new-token queries.
 *   k_cache,
 *   v_cache     [cu_seqlens[batch], hkv, dh] packed caches (rotated keys).
 *   g           [cu_seqlens[batch]] fp32 gate values, or NULL for no bias.
 *   head_gain   [hq] fp32 gamma_h, or NULL for 1.
 *   o           [batch, hq, dh] output, dtype.   lse: [batch, hq] fp32 or NULL.
 *   workspace   device memory owned by the caller, 16-byte aligned, at least
 *               tg_decode_attn_workspace_size(...) bytes: partial results of
 *               the key blocks; contents need not be initialised and are
 *               left undefined.  Calls that share a workspace must not
 *               overlap.  The library allocates nothing.
 * Errors: TG_ERR_INVALID_ARG for NULL pointers, misalignment or out-of-range
 * sizes; TG_ERR_WORKSPACE for a workspace smaller than the size function
 * returns; TG_ERR_UNSUPPORTED for other head ratios or dh; TG_ERR_HIP for a
 * failed launch.  batch = 0 is a no-op.
 * ------------------------------------------------------------------------- */
TG_API int64_t tg_decode_attn_workspace_size(int32_t batch, int64_t max_seqlen, int32_t hq,
                                             int32_t hkv, int32_t dh);
TG_API tg_status tg_decode_attn(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh,
                                float scale, const void* q, const void* k_cache,
                                const void* v_cache, const float* g, const float* head_gain,
                                void* o, float* lse, void* workspace, int64_t workspace_bytes,
                                hipStream_t stream);

/* Decode attention for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation, arguments and errors as tg_decode_attn, with no workspace
 * argument: the split-K partial results go to a file-scope device array of
 * tg_decode_attn_noalloc_max_bytes() bytes (16 MiB), which each GPU the
 * library runs on holds until the process ends.  The call allocates nothing;
 * its first call on a device looks up that device's copy of the array (with
 * the device current: `stream` must belong to the current device).
 *  - A request whose workspace (tg_decode_attn_workspace_size) exceeds the
 *    array returns TG_ERR_WORKSPACE before any HIP call.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero): calls that
 *    overlap on one GPU (different streams, or threads) race.  Order them.
 * The array is global state of the library, the one exception to the
 * convention above. */
TG_API int64_t tg_decode_attn_noalloc_max_bytes(void);
TG_API tg_status tg_decode_attn_noalloc(tg_dtype dtype, const int32_t* cu_seqlens, int32_t batch,
                                        int64_t max_seqlen, int32_t hq, int32_t hkv, int32_t dh,
                                        float scale, const void* q, const void* k_cache,
                                        const void* v_cache, const float* g, const float* head_gain,
                                        void* o, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Upper-layer dense work on the kept tokens.  [aitu] section 3: every layer
 * above the selection layer processes only the kept tokens, so its
 * projections and MLP are products of the [K, d] kept activations with the
 * layer's weights.  Layer shape: the base model of the [paper] setup table
 * (Qwen3-1.7B, bf16): bias-free QKV / O projections and a SwiGLU MLP.  The
 * setup's LoRA adapters (rank 16, alpha 32, query and value projections) are
 * taken as merged into W before the path (W + (alpha/r) B A).
 *
 * tg_linear:  y = x W^T            (residual NULL)
 *             y = x W^T + residual  (residual may equal y, with ld_r == ld_y:
 *                                    in-place add)
 * tg_swiglu:  y = SiLU(x Wg^T) * (x Wu^T),  SiLU(z) = z / (1 + e^-z)
 * The MLP block is tg_swiglu followed by tg_linear with W_down and the
 * residual stream.
 *
 *   dtype     TG_BF16 only (TG_FP32 gives TG_ERR_UNSUPPORTED): bf16 operands,
 *             fp32 accumulation (MFMA), one bf16 rounding of the result (after
 *             the residual add / the SwiGLU product).
 *   m         rows (tokens), 0 <= m < 2^31 (0 is a no-op).
 *   n         output columns of tg_linear, a multiple of 256.
 *   f         output columns of tg_swiglu, a multiple of 128.
 *   k         inner size, a multiple of 32.
 *   x         [m, ld_x] bf16, row-major, 16-byte aligned, ld_x >= k, ld_x % 8 == 0.
 *   w         [n, ld_w] bf16 (nn.Linear layout: one output per row),
 *             16-byte aligned, ld_w >= k, ld_w % 8 == 0.  w_gate, w_up: [f, ld_w].
 *   residual  [m, ld_r] bf16 or NULL.
 *   y         [m, ld_y] bf16, ld_y >= n (or f).  Must not overlap x or w.
 * Errors: TG_ERR_INVALID_ARG for NULL pointers, misalignment, bad leading
 * dimensions or sizes out of range; TG_ERR_UNSUPPORTED for other dtypes and
 * for n, f, k off the multiples above; TG_ERR_HIP for a failed launch.
 * ------------------------------------------------------------------------- */
TG_API tg_status tg_linear(tg_dtype dtype, int64_t m, int32_t n, int32_t k, const void* x,
                           int64_t ld_x, const void* w, int64_t ld_w, const void* residual,
                           int64_t ld_r, void* y, int64_t ld_y, hipStream_t stream);
TG_API tg_status tg_swiglu(tg_dtype dtype, int64_t m, int32_t f, int32_t k, const void* x,
                           int64_t ld_x, const void* w_gate, const void* w_up, int64_t ld_w,
                           void* y, int64_t ld_y, hipStream_t stream);

/* The fused QKV projection of an upper layer: one product with the stacked
 * weight w_qkv = [Wq; Wk; Wv] ([(hq + 2 hkv) dh, ld_w], nn.Linear layout) whose
 * output columns go straight to the three buffers tg_rope_kv and the
 * attention read:  q [m, hq, dh], k_out [m, hkv, dh], v_out [m, hkv, dh]
 * (contiguous, bf16).  hq*dh and hkv*dh must be multiples of 256; other
 * arguments and errors as tg_linear (n = (hq + 2 hkv) dh). */
TG_API tg_status tg_qkv_proj(tg_dtype dtype, int64_t m, int32_t hq, int32_t hkv, int32_t dh,
                             int32_t k, const void* x, int64_t ld_x, const void* w_qkv,
                             int64_t ld_w, void* q, void* k_out, void* v_out,
                             hipStream_t stream);

/* Check of the position precondition of the attention entry points (the
 * pages' causal mask is on original positions; with strictly increasing
 * positions it equals the mask on kept indices, which the attention kernels
 * of both dtypes use).
 * Writes to *first_bad (device int32) the smallest row i that breaks the
 * order -- pos[i] < 0, or pos[i] <= pos[i-1] with row i-1 in the same
 * sequence -- or `total` when every row is in order.  cu_seqlens [batch+1]
 * (device) splits the rows into sequences as in tg_gated_attn_varlen, or NULL
 * for one sequence.  Two small kernels on `stream`; no synchronisation, no
 * allocation.  Errors: TG_ERR_INVALID_ARG for NULL pointers or sizes out of
 * range. */
TG_API tg_status tg_check_positions(const int32_t* pos, int64_t total, const int32_t* cu_seqlens,
                                    int32_t batch, int32_t* first_bad, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H_ */
