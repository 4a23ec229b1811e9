// Internal declarations shared by the HIP translation units of libtokengate.
// Not part of the public ABI (see include/tokengate.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// ---- vector types used with the gfx950 MFMA builtins ----------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFltMin = 1.17549435e-38f;  // smallest normal fp32, 2^-126

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// 16-byte global -> LDS copy (global_load_lds_dwordx4): lane l's bytes land at
// LDS address m0 + 16 l.  Written as asm so that the compiler's wait-count
// pass does not track it: once copies stay in flight across a loop back-edge
// that pass loses track of which LDS buffer they target and drains all of
// them before any LDS read.  The instruction has no register results; the
// caller orders completion with explicit vmcnt waits (wait_vm).  A
// compiler-visible global load issued while such copies are in flight gets a
// wait that also drains them, so loops built on dma16 keep all other global
// loads outside the pipelined region.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr) : "memory");
}

// 4-byte copy: lane l's dword lands at lds_addr + 4 l.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_addr) : "memory");
}

// Same copy from a wave-uniform 64-bit base (scalar registers) plus a 32-bit
// per-lane byte offset: one vector register per copy instead of two.
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// s_waitcnt immediate (gfx9 layout) that waits for vmcnt <= v, nothing else.
template <int V>
__device__ __forceinline__ void wait_vm() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (V & 15) | ((V >> 4) << 14));
}

// Workgroup barrier without the release/acquire fence of __syncthreads: the
// fence would wait for every outstanding global->LDS copy.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// One dispatch counts work-items in 32 bits in x and allows 65535 blocks in
// y and z.  Launchers refuse larger grids before any HIP call with
// hipErrorInvalidConfiguration, which the C ABI reports as TG_ERR_UNSUPPORTED.
constexpr int64_t kMaxGridItemsX = 0xffffffffLL;
constexpr int64_t kMaxGridBlocksYZ = 65535;
inline bool grid_fits(int64_t blocks_x, int threads, int64_t y = 1, int64_t z = 1) {
  return blocks_x >= 0 && blocks_x <= kMaxGridItemsX / threads && y >= 0 && y <= kMaxGridBlocksYZ && z >= 0 &&
         z <= kMaxGridBlocksYZ;
}

// ---- launchers (defined in the kernel translation units) -------------------
hipError_t launch_gate_bf16(int64_t n, int d, int hidden, const void* h, int64_t ld_h,
                            const void* w1, const float* b1, const float* w2, float b2,
                            float* g, float* s, hipStream_t stream);
// Gate MLP whose last workgroup also ranks the scores it wrote (bf16 only;
// select workspace zero on entry, zero again on exit), then the compaction
// kernel: idx, and with h_out the kept rows, gate values and positions.
// Requires 0 < kd = min(k, n) - q_len < n - q_len and a document of at most
// gate_select_block_tokens(hidden) tokens (what the last workgroup holds in
// LDS; longer documents take the gate, the multi-workgroup select and the
// gather instead).
int64_t gate_select_block_tokens(int hidden);
hipError_t launch_gate_select_bf16(int64_t n, int d, int hidden, const void* h, int64_t ld_h, const void* w1,
                                   const float* b1, const float* w2, float b2, float* g, float* s, int64_t k,
                                   int64_t q_len, int32_t* idx, void* workspace, void* h_out, float* g_out,
                                   int32_t* pos_out, hipStream_t stream);
hipError_t launch_gate_f32(int64_t n, int d, int hidden, const float* h, int64_t ld_h,
                           const float* w1, const float* b1, const float* w2, float b2,
                           float* g, float* s, hipStream_t stream);

// Several workgroups per prompt (select.hip), with a caller workspace of
// select_mw_workspace_bytes(n) bytes.  ws_clean: the workspace is known to be
// zero (as every call leaves it); otherwise a small kernel clears it first.
int64_t select_mw_workspace_bytes(int64_t n);
hipError_t launch_select_mw(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx, void* workspace,
                            bool ws_clean, hipStream_t stream);
// Compaction after a multi-workgroup ranking (T, need and the chunk counts in
// the workspace): idx, and with h_out != NULL also the kept rows of h
// (row_bytes each, ld_h_bytes apart), their gate values and positions.
hipError_t launch_compact(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx, const void* workspace,
                          const void* h, int64_t ld_h_bytes, int row_bytes, void* h_out, float* g_out,
                          int32_t* pos_out, hipStream_t stream);
hipError_t launch_select(const float* g, int64_t n, int64_t k, int64_t q_len,
                         const int32_t* cu_seqlens, const int32_t* q_lens, int batch,
                         int64_t max_seqlen, int32_t* idx, int32_t* cu_kept,
                         hipStream_t stream);

hipError_t launch_gather(int elem_bytes, int64_t n, int64_t n_kept, int d, const int32_t* idx,
                         const void* h, int64_t ld_h, const float* g, void* h_out,
                         float* g_out, int32_t* pos_out, const int32_t* cu_seqlens,
                         const int32_t* cu_kept, int batch, int64_t max_kept,
                         hipStream_t stream);

hipError_t launch_rope_table(float* cos_sin, int64_t max_pos, int dh, double base,
                             hipStream_t stream);
hipError_t launch_rope_kv(int elem_bytes, int64_t n_kept, int hq, int hkv, int dh,
                          const int32_t* pos, const float* cos_sin, int64_t max_pos, void* q,
                          const void* k, const void* v, void* k_cache, void* v_cache,
                          hipStream_t stream);

hipError_t launch_attn_bf16(int64_t total, const int32_t* cu_seqlens, int batch,
                            int64_t max_seqlen, int hq, int hkv, int dh, float scale,
                            const void* q, const void* k, const void* v, const float* g,
                            const float* head_gain, const int32_t* pos, void* o, float* lse,
                            hipStream_t stream);
hipError_t launch_attn_f32(int64_t total, const int32_t* cu_seqlens, int batch,
                           int64_t max_seqlen, int hq, int hkv, int dh, float scale,
                           const float* q, const float* k, const float* v, const float* g,
                           const float* head_gain, float* o, float* lse,
                           hipStream_t stream);

// Decode attention: keys per split-K block, and the launch of the split and
// combine kernels (workspace: batch * hq * nsplit * (dh + 2) floats).
int decode_split_keys(int64_t batch, int hkv, int64_t max_seqlen);
// The decode workspace of the entry point that allocates nothing: a
// file-scope device array of this many bytes in decode.hip, and the device
// address of the current device's copy (looked up once per device).
constexpr int64_t kDecodeStaticScratchBytes = int64_t(16) << 20;
hipError_t decode_static_scratch(void** ptr);
hipError_t launch_decode(int elem_bytes, const int32_t* cu_seqlens, int batch, int64_t max_seqlen, int hq,
                         int hkv, int dh, float scale, const void* q, const void* k, const void* v,
                         const float* g, const float* head_gain, void* o, float* lse, float* workspace,
                         hipStream_t stream);

// Writes the smallest row whose position breaks the strictly-increasing,
// non-negative order within its sequence, or `total`.
hipError_t launch_check_positions(const int32_t* pos, int64_t total, const int32_t* cu_seqlens, int batch,
                                  int32_t* first_bad, hipStream_t stream);

// Dense product C = A W^T on bf16 with an epilogue: 0 plain, 1 residual add,
// 2 SwiGLU (w = gate weights, w2 = up weights, n = F).
hipError_t launch_gemm_bf16(int epi, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const void* w,
                            const void* w2, int64_t ldw, const void* r, int64_t ldr, void* c, int64_t ldc,
                            hipStream_t stream);
// Same, plain epilogue only, with the output columns split over three buffers:
// [0, s1) -> c, [s1, s2) -> c1, [s2, n) -> c2 (s1, s2 multiples of 256).
hipError_t launch_gemm_bf16_split(int epi, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                                  const void* w, const void* w2, int64_t ldw, const void* r, int64_t ldr, void* c,
                                  int64_t ldc, void* c1, int64_t ld1, int64_t s1, void* c2, int64_t ld2, int64_t s2,
                                  hipStream_t stream);

}  // namespace tg
