// Stage 1 -- TokenGate's gate MLP on gfx950.
//
// TokenGate paper page (thelatestinai.com), Figure 1(b): a small scoring
// network scores every hidden state at the selection layer; aitualizate.com
// article, section "2. Una red MLP aprende qué tokens conservar": the MLP
// reads each token's post-attention residual state.  Form used here:
//   g_j = sigmoid(b2 + sum_k w2_k * SiLU(b1_k + sum_i W1[k,i] h[j,i])).
//
// bf16 kernel: one workgroup = 128 tokens x all `hidden` units, so the w2 dot
// and the sigmoid finish inside the workgroup with no second pass.  The
// h-by-W1^T product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// h and W1 are staged through LDS in 64-element k-chunks, double-buffered,
// with the next chunk prefetched into registers while the current one feeds
// the matrix cores.  The hidden layer never leaves fp32 registers.
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kGateBM = 128;       // tokens per workgroup
constexpr int kGateBK = 64;        // k elements per LDS stage (128 bytes of a row)
constexpr int kGateThreads = 256;  // 4 waves: 2 along tokens x 2 along hidden units

// LDS tile rows are 128 bytes = 8 chunks of 16 bytes.  Chunk c of row r is
// stored at chunk slot c ^ ((r >> 1) & 7): the 16 rows read by one
// ds_read_b128 quarter-wave then hit all 64 banks exactly once.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int H>
__global__ __launch_bounds__(kGateThreads) void gate_bf16_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int n, int d, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2, float* __restrict__ g,
    float* __restrict__ s_out) {
  constexpr int MT = 2;               // 32-token tiles per wave
  constexpr int NT = H / 2 / 32;      // 32-unit tiles per wave
  constexpr int A_LOADS = kGateBM * 8 / kGateThreads;  // 16-byte chunks per thread (h)
  constexpr int B_LOADS = H * 8 / kGateThreads;        // 16-byte chunks per thread (W1)
  constexpr int STAGE = (kGateBM + H) * 128;           // bytes per LDS stage

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  __shared__ float srow[2][kGateBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // token half
  const int wn = wave >> 1;  // hidden-unit half
  const int m0 = blockIdx.x * kGateBM;

  // Per-thread load coordinates: chunk (16 bytes) and row within the tile.
  const int lchunk = tid & 7;
  const int lrow = tid >> 3;  // 0..31, +32 per load

  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w1);

  u32x4 ra[A_LOADS];
  u32x4 rb[B_LOADS];

  auto load_regs = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      int row = m0 + lrow + 32 * i;
      row = row < n ? row : n - 1;  // rows past n read a valid row, results discarded
      ra[i] = *reinterpret_cast<const u32x4*>(hb + ((int64_t)row * ld_h + k0) * 2 + lchunk * 16);
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int row = lrow + 32 * i;
      rb[i] = *reinterpret_cast<const u32x4*>(wb + ((int64_t)row * d + k0) * 2 + lchunk * 16);
    }
  };
  auto store_lds = [&](int stage) {
    uint8_t* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      *reinterpret_cast<u32x4*>(base + swz(lrow + 32 * i, lchunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      *reinterpret_cast<u32x4*>(base + kGateBM * 128 + swz(lrow + 32 * i, lchunk)) = rb[i];
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = d / kGateBK;
  load_regs(0);
  store_lds(0);
  __syncthreads();

  const int half = lane >> 5;   // which 8-element k group of the MFMA operand
  const int r32 = lane & 31;

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_regs((kt + 1) * kGateBK);
    const uint8_t* base = lds + (kt & 1) * STAGE;
#pragma unroll
    for (int ks = 0; ks < kGateBK / 16; ++ks) {
      const int chunk = ks * 2 + half;
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(base + swz(wm * 64 + i * 32 + r32, chunk));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(base + kGateBM * 128 +
                                                  swz(wn * (H / 2) + j * 32 + r32, chunk));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue.  acc[i][j][r] holds token  wm*64 + i*32 + 8*(r/4) + 4*half + r%4
  // and hidden unit  wn*H/2 + j*32 + r32.
  float part[MT][16];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[i][r] = 0.0f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int unit = wn * (H / 2) + j * 32 + r32;
    const float bias = b1 ? b1[unit] : 0.0f;
    const float wout = w2[unit];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = acc[i][j][r] + bias;
        const float z = a / (1.0f + expf(-a));  // SiLU
        part[i][r] = fmaf(wout, z, part[i][r]);
      }
  }
  // Sum over the 32 lanes that share a token (same `half`).
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = part[i][r];
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
      part[i][r] = v;
    }
  if (r32 == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        srow[wn][wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = part[i][r];
  }
  __syncthreads();
  if (tid < kGateBM) {
    const int row = m0 + tid;
    if (row < n) {
      const float sc = srow[0][tid] + srow[1][tid] + b2;
      g[row] = 1.0f / (1.0f + expf(-sc));
      if (s_out) s_out[row] = sc;
    }
  }
}

// fp32 gate: one wave per token, lanes stride over hidden units.
__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ h, int64_t ld_h,
                                                       int n, int d, int hidden,
                                                       const float* __restrict__ w1,
                                                       const float* __restrict__ b1,
                                                       const float* __restrict__ w2, float b2,
                                                       float* __restrict__ g,
                                                       float* __restrict__ s_out) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= n) return;
  const f32x4* hr = reinterpret_cast<const f32x4*>(h + tok * ld_h);
  float part = 0.0f;
  for (int u = lane; u < hidden; u += kWave) {
    const f32x4* wr = reinterpret_cast<const f32x4*>(w1 + (int64_t)u * d);
    float a = 0.0f;
    for (int i = 0; i < d / 4; ++i) {
      const f32x4 x = hr[i];
      const f32x4 w = wr[i];
      a = fmaf(x[0], w[0], a);
      a = fmaf(x[1], w[1], a);
      a = fmaf(x[2], w[2], a);
      a = fmaf(x[3], w[3], a);
    }
    if (b1) a += b1[u];
    const float z = a / (1.0f + expf(-a));
    part = fmaf(w2[u], z, part);
  }
  const float sc = wave_sum(part) + b2;
  if (lane == 0) {
    g[tok] = 1.0f / (1.0f + expf(-sc));
    if (s_out) s_out[tok] = sc;
  }
}

}  // namespace

hipError_t launch_gate_bf16(int64_t n, int d, int hidden, const void* h, int64_t ld_h,
                            const void* w1, const float* b1, const float* w2, float b2, float* g,
                            float* s, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kGateBM - 1) / kGateBM));
  const auto* hh = static_cast<const uint16_t*>(h);
  const auto* ww = static_cast<const uint16_t*>(w1);
  switch (hidden) {
    case 64:
      hipLaunchKernelGGL(gate_bf16_kernel<64>, grid, dim3(kGateThreads), 0, stream, hh, ld_h, (int)n,
                         d, ww, b1, w2, b2, g, s);
      break;
    case 128:
      hipLaunchKernelGGL(gate_bf16_kernel<128>, grid, dim3(kGateThreads), 0, stream, hh, ld_h,
                         (int)n, d, ww, b1, w2, b2, g, s);
      break;
    default:
      hipLaunchKernelGGL(gate_bf16_kernel<256>, grid, dim3(kGateThreads), 0, stream, hh, ld_h,
                         (int)n, d, ww, b1, w2, b2, g, s);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_f32(int64_t n, int d, int hidden, const float* h, int64_t ld_h,
                           const float* w1, const float* b1, const float* w2, float b2, float* g,
                           float* s, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 3) / 4));
  hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(256), 0, stream, h, ld_h, (int)n, d, hidden, w1, b1,
                     w2, b2, g, s);
  return hipGetLastError();
}

}  // namespace tg
