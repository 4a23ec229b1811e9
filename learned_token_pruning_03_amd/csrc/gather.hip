// Stage 3 -- gather of the kept tokens, on gfx950.
//
// TokenGate paper page (thelatestinai.com), Figure 1(b): the top-K selector
// forwards the kept hidden states together with their importance scores;
// aitualizate.com article, section "3. Las capas superiores procesan
// únicamente los tokens seleccionados": only the kept tokens go up.  Each
// kept token also carries its original position, so that the upper layers
// can apply RoPE and the causal mask at the token's place in the prompt.
//
// A pure bandwidth kernel: one wave per kept row, 16-byte loads and stores,
// every load of a row issued before its stores.
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void gather_kernel(
    int64_t n, int64_t n_kept, int row_chunks, const int32_t* __restrict__ idx,
    const uint8_t* __restrict__ h, int64_t ld_bytes, const float* __restrict__ g,
    uint8_t* __restrict__ h_out, float* __restrict__ g_out, int32_t* __restrict__ pos_out,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_kept) {
  const int lane = threadIdx.x & 63;
  const int64_t local = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  int64_t lo = 0, hi = n_kept, row0 = 0, nrows = n;
  if (cu_kept) {  // packed batch: blockIdx.y is the prompt
    const int b = blockIdx.y;
    lo = cu_kept[b];
    hi = cu_kept[b + 1];
    row0 = cu_seqlens[b];
    nrows = cu_seqlens[b + 1] - row0;
  }
  const int64_t i = lo + local;
  if (i >= hi) return;
  const int32_t p = idx[i];
  const bool ok = p >= 0 && p < nrows;
  const uint8_t* src = h + (row0 + (ok ? p : 0)) * ld_bytes;
  uint8_t* dst = h_out + i * (int64_t)row_chunks * 16;

  for (int c0 = 0; c0 < row_chunks; c0 += kWave * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < row_chunks) v[u] = ok ? *reinterpret_cast<const u32x4*>(src + c * 16) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < row_chunks) *reinterpret_cast<u32x4*>(dst + c * 16) = v[u];
    }
  }
  if (lane == 0) {
    if (g_out) g_out[i] = ok ? g[row0 + p] : 0.0f;
    if (pos_out) pos_out[i] = ok ? p : -1;
  }
}

}  // namespace

hipError_t launch_gather(int elem_bytes, int64_t n, int64_t n_kept, int d, const int32_t* idx,
                         const void* h, int64_t ld_h, const float* g, void* h_out, float* g_out,
                         int32_t* pos_out, const int32_t* cu_seqlens, const int32_t* cu_kept,
                         int batch, int64_t max_kept, hipStream_t stream) {
  const int row_chunks = (int)((int64_t)d * elem_bytes / 16);
  const int64_t rows = cu_kept ? max_kept : n_kept;
  if (!grid_fits((rows + kRowsPerBlock - 1) / kRowsPerBlock, 256, cu_kept ? batch : 1))
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), cu_kept ? (unsigned)batch : 1u);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, stream, n, n_kept, row_chunks, idx,
                     static_cast<const uint8_t*>(h), ld_h * elem_bytes, g,
                     static_cast<uint8_t*>(h_out), g_out, pos_out, cu_seqlens, cu_kept);
  return hipGetLastError();
}

// ---- check of the attention entry points' position precondition ---------
// Within each sequence the positions must be non-negative and strictly
// increasing (the order select + gather produce).  The first kernel sets the
// answer to `total` (no offending row); the second lowers it to the smallest
// offending row with a vector atomic.
namespace {

__global__ __launch_bounds__(64) void check_pos_init_kernel(int32_t* bad, int32_t total) {
  if (threadIdx.x == 0) *bad = total;
}

__global__ __launch_bounds__(256) void check_pos_kernel(const int32_t* __restrict__ pos, int32_t total,
                                                        const int32_t* __restrict__ cu, int32_t batch,
                                                        int32_t* bad) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  bool first = i == 0;
  if (cu && !first) {  // largest b with cu[b] <= i; row i starts a sequence iff cu[b] == i
    int lo = 0, hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= i)
        lo = mid;
      else
        hi = mid - 1;
    }
    first = cu[lo] == i;
  }
  const int32_t p = pos[i];
  if (p < 0 || (!first && p <= pos[i - 1])) atomicMin(bad, (int32_t)i);
}

}  // namespace

hipError_t launch_check_positions(const int32_t* pos, int64_t total, const int32_t* cu_seqlens, int batch,
                                   int32_t* first_bad, hipStream_t stream) {
  if (!grid_fits((total + 255) / 256, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(check_pos_init_kernel, dim3(1), dim3(64), 0, stream, first_bad, (int32_t)total);
  if (total > 0)
    hipLaunchKernelGGL(check_pos_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, pos,
                       (int32_t)total, cu_seqlens, batch, first_bad);
  return hipGetLastError();
}

}  // namespace tg
