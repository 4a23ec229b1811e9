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
// h-by-W1^T product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// h and W1 stream through LDS in 64-element k-chunks over a three-stage ring
// filled by global_load_lds (no register staging), so two chunks are always in
// flight while the matrix cores consume the third; h is read from HBM once.
// Eight waves, two per SIMD: waves w and w+4 own the same 64-token x H/2-unit
// output tile and take alternate 16-wide k sub-steps, so one wave's MFMAs
// cover the other's LDS and DMA waits.  The two partial sums meet in LDS
// before the SiLU epilogue, which the pair also splits.  The hidden layer
// never leaves fp32 registers.
// Each workgroup walks the k-chunks in its own rotated order.  Workgroups
// are dealt to the eight XCDs in turn, so workgroup b starts at chunk
// (b / 8) mod (d / 64): the workgroups of one XCD then read 128-byte pieces
// at different column offsets of their rows at any moment, and the h stream
// reaches about the rate of a contiguous copy.  All starting at chunk 0, the
// same stream runs ~30% slower.
#include <type_traits>

#include "select_core.h"

namespace tg {
namespace {

constexpr int kGateBM = 128;       // tokens per workgroup
constexpr int kGateBK = 64;        // k elements per LDS stage (128 bytes of a row)
constexpr int kGateThreads = 512;  // 8 waves: 2 along tokens x 2 along hidden units x 2 along k

// Bytes of one stage of the LDS ring (an h tile and a W1 tile, 128-byte
// rows), and the document keys the last workgroup of the selecting form can
// hold in the ring's three stages once the ring is free.
template <int H>
struct GateRing {
  static constexpr int kStage = kGateBM * 128 + H * 128;
  static constexpr int kPage = kStage / 4 / kCompactChunk * kCompactChunk;
  static constexpr int kBlockTok =
      3 * kPage < kSelMaxBlockChunks * kCompactChunk ? 3 * kPage : kSelMaxBlockChunks * kCompactChunk;
  static_assert(kPage % 256 == 0 && kBlockTok % 256 == 0, "keys are copied in 256-key blocks");
};

// LDS tile rows are 128 bytes = 8 chunks of 16 bytes.  Chunk c of row r is
// stored at chunk slot c ^ ((r >> 1) & 7): the 16 rows read by one
// ds_read_b128 quarter-wave then hit all 64 banks exactly once.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Selection arguments of the fused form (SEL): document length, document
// tokens to keep and the select workspace.
struct GateSel {
  int doc, kd;
  uint32_t* ws;
};

template <int H, bool SEL>
__global__ __launch_bounds__(kGateThreads) void gate_bf16_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int n, int d, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2, float* __restrict__ g,
    float* __restrict__ s_out, GateSel sel) {
  constexpr int NW = kGateThreads / kWave;            // 8 waves
  constexpr int MT = 2;                               // 32-token tiles per wave
  constexpr int NT = H / 2 / 32;                      // 32-unit tiles per wave
  constexpr int A_DMA = kGateBM * 8 / kGateThreads;   // 16-byte chunks per thread per stage (h)
  constexpr int B_DMA = H * 8 / kGateThreads;         // same for W1
  constexpr int PER_CHUNK = A_DMA + B_DMA;            // vmcnt increments per stage per wave
  constexpr int H_BYTES = kGateBM * 128;
  constexpr int STAGE = GateRing<H>::kStage;
  static_assert(A_DMA >= 1 && B_DMA >= 1 && (MT * NT) % 2 == 0, "tile shape");

  // Three separate objects, so the compiler can tell that reads of one stage
  // do not depend on the DMA still landing in the other two.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];
  __shared__ float srow[4][kGateBM];
  // Ranking state of the fused form (the keys themselves go to the ring).
  __shared__ std::conditional_t<SEL, SelFinishShared, char> sel_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave & 3;  // output tile shared by waves w and w+4
  const int kh = wave >> 2;   // which 16-wide k sub-steps of each chunk this wave takes
  const int wm = tile & 1;    // token half
  const int wn = tile >> 1;   // hidden-unit half
  const int m0 = blockIdx.x * kGateBM;

  // DMA mapping: instruction i of wave w fills the 1 KB block b = NW i + w of
  // a region; lane l lands at byte 16 l of it, i.e. row 8 b + l/8, slot l%8,
  // which holds chunk (l%8) ^ ((row >> 1) & 7).
  const uint8_t* pa[A_DMA];
  const uint8_t* pb[B_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const int r = (NW * i + wave) * 8 + (lane >> 3);
    int row = m0 + r;
    row = row < n ? row : n - 1;  // rows past n read a valid row, results discarded
    pa[i] = reinterpret_cast<const uint8_t*>(h) + (int64_t)row * ld_h * 2 +
            (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    const int r = (NW * i + wave) * 8 + (lane >> 3);
    pb[i] = reinterpret_cast<const uint8_t*>(w1) + (int64_t)r * d * 2 +
            (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }

  // Step kt of the k loop reads chunk (kt + k_rot) mod nk.
  const int nk = d / kGateBK;
  const int k_rot = (int)((blockIdx.x / 8) % (unsigned)nk);
  // Copy q of this wave for loop step kt into stage sb: h blocks first, then W1.
  auto issue_one = [&](int q, int kt, uint8_t* sb) __attribute__((always_inline)) {
    const int kc = kt + k_rot < nk ? kt + k_rot : kt + k_rot - nk;
    const int koff = kc * (kGateBK * 2);
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)sb;
    if (q < A_DMA)
      dma16(pa[q] + koff, base + (NW * q + wave) * 1024);
    else
      dma16(pb[q - A_DMA] + koff, base + H_BYTES + (NW * (q - A_DMA) + wave) * 1024);
  };
  auto issue = [&](int kt, uint8_t* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PER_CHUNK; ++q) issue_one(q, kt, sb);
  };
  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int half = lane >> 5;  // which 8-element k group of the MFMA operand
  const int r32 = lane & 31;
  // b1 and w2 at this lane's hidden units, for the epilogue.  Loaded here,
  // ahead of the first copies, so that they have long arrived when the
  // epilogue needs them (loaded there, each tile waited for its own loads).
  float bias_u[NT], wout_u[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int unit = wn * (H / 2) + j * 32 + r32;
    bias_u[j] = b1 ? b1[unit] : 0.0f;
    wout_u[j] = w2[unit];
  }

  // This wave takes sub-steps 2 kh and 2 kh + 1 of every 64-wide chunk; its
  // partner (same tile, other kh) takes the other two.  Both fragment sets are
  // read before the first MFMA; the second wave on the SIMD covers the wait.
  // The copies of chunk kt_next (if any) are spread between the MFMAs, one
  // after every second MFMA: issued all at once, the eight waves' copies queue
  // up in the address unit and hold back the MFMAs of the later waves.
  auto compute = [&](const uint8_t* base, int kt_next, uint8_t* sb_next) __attribute__((always_inline)) {
    bf16x8 af[2][MT], bfr[2][NT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int chunk = (2 * kh + u) * 2 + half;
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[u][i] = *reinterpret_cast<const bf16x8*>(base + swz(wm * 64 + i * 32 + r32, chunk));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[u][j] = *reinterpret_cast<const bf16x8*>(base + H_BYTES + swz(wn * (H / 2) + j * 32 + r32, chunk));
    }
    const bool copy = kt_next >= 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int mi = (u * MT + i) * NT + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u][i], bfr[u][j], acc[i][j], 0, 0, 0);
          if ((mi & 1) && (mi >> 1) < PER_CHUNK) {
            __builtin_amdgcn_sched_barrier(0);
            if (copy) issue_one(mi >> 1, kt_next, sb_next);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
    for (int q = MT * NT; q < PER_CHUNK; ++q)  // copies left over when there are few MFMAs
      if (copy) issue_one(q, kt_next, sb_next);
  };

  // One ring step: chunk kt sits in stage `cur`; chunk kt+2 goes to `nxt2`,
  // the stage every wave finished reading in the previous step.
  auto step = [&](int kt, const int nk, uint8_t* cur, uint8_t* nxt2) __attribute__((always_inline)) {
    if (kt + 1 < nk)
      wait_vm<PER_CHUNK>();  // chunk kt+1 may still be landing
    else
      wait_vm<0>();
    // Every wave has waited for its own share of chunk kt; chunks kt+1 and
    // kt+2 stay in flight across the barrier.
    plain_barrier();
    compute(cur, kt + 2 < nk ? kt + 2 : -1, nxt2);
  };

  issue(0, st0);
  if (nk > 1) issue(1, st1);
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, nk, st0, st2);
    step(kt + 1, nk, st1, st0);
    step(kt + 2, nk, st2, st1);
  }
  if (kt < nk) step(kt, nk, st0, st2);
  if (kt + 1 < nk) step(kt + 1, nk, st1, st0);

  // ---- combine the two k halves, then the epilogue, split between partners.
  // Of the MT*NT output tiles, tile t = i*NT + j stays with the wave whose kh
  // equals t%2; the other half goes to the partner (wave ^ 4) through LDS.
  // The ring is free once every wave has passed the barrier below.
  constexpr int KEEP = MT * NT / 2;                 // tiles per wave after the split
  constexpr int XBYTES = KEEP * 16 * kWave * 4;     // bytes one wave hands over
  constexpr int PER_STAGE = STAGE / XBYTES;
  static_assert(3 * PER_STAGE >= NW, "exchange fits in the ring");
  auto region = [&](int w) __attribute__((always_inline)) {
    const int sidx = w / PER_STAGE;
    uint8_t* sb = sidx == 0 ? st0 : (sidx == 1 ? st1 : st2);
    return reinterpret_cast<f32x4*>(sb + (w % PER_STAGE) * XBYTES);
  };
  __syncthreads();
  {
    f32x4* out = region(wave);
    int q = 0;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (((i * NT + j) & 1) != kh) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            out[(q * 4 + r4) * kWave + lane] = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1],
                                                acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
          ++q;
        }
  }
  __syncthreads();

  // acc[i][j][r] holds token  wm*64 + i*32 + 8*(r/4) + 4*half + r%4  and
  // hidden unit  wn*H/2 + j*32 + r32.
  float part[MT][16];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[i][r] = 0.0f;
  {
    const f32x4* in = region(wave ^ 4);
    int q = 0;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (((i * NT + j) & 1) == kh) {
          const float bias = bias_u[j];
          const float wout = wout_u[j];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 o = in[(q * 4 + r4) * kWave + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a = acc[i][j][4 * r4 + e] + o[e] + bias;
              // SiLU(a) = a / (1 + e^-a) with the hardware exp2 and reciprocal.
              const float ex = __builtin_amdgcn_exp2f(-a * kLog2e);
              const float z = a * __builtin_amdgcn_rcpf(1.0f + ex);
              part[i][4 * r4 + e] = fmaf(wout, z, part[i][4 * r4 + e]);
            }
          }
          ++q;
        }
  }
  // Sum over the 32 lanes that share a token (same `half`), on the DPP lane
  // network: within each 16-lane row, adds across lane pairs (xor 1), lane
  // pairs of quads (xor 2), mirrored half-rows and mirrored rows leave the
  // row's sum in all its lanes; then every row adds lane 15 of the row before
  // it (row_bcast:15), so lanes 31 and 63 hold the sums of their halves.  Each
  // step is an add with a DPP source (the broadcast a DPP move and an add); a
  // shuffle per step would go through the LDS and wait for it.
  auto dpp_add = [](float v, auto ctrl_tag) __attribute__((always_inline)) {
    constexpr int ctrl = decltype(ctrl_tag)::value;
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, true));
  };
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = part[i][r];
      v = dpp_add(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
      v = dpp_add(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
      v = dpp_add(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
      v = dpp_add(v, std::integral_constant<int, 0x140>{});  // row_mirror
      v = dpp_add(v, std::integral_constant<int, 0x142>{});  // row_bcast:15 (rows 0 and 2 unused after it)
      part[i][r] = v;
    }
  if (r32 == 31) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        srow[wn * 2 + kh][wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = part[i][r];
  }
  __syncthreads();
  if constexpr (SEL) {
    for (int i = tid; i < kSelBins; i += kGateThreads) sel_sh.hist[i] = 0u;
  }
  float gv = 0.0f;
  const int row = m0 + tid;
  if (tid < kGateBM && row < n) {
    const float sc = (srow[0][tid] + srow[1][tid]) + (srow[2][tid] + srow[3][tid]) + b2;
    gv = 1.0f / (1.0f + expf(-sc));
    g[row] = gv;
    if (s_out) s_out[row] = sc;
  }
  if constexpr (SEL) {
    // TokenGate paper page, Figure 1(b): the selector ranks the scores the
    // gate just produced.  Top-digit counts of this workgroup's document
    // tokens go to the workspace; the last workgroup to finish selects.
    // The order keys go to the workspace too, written past the L2: the last
    // workgroup copies them into LDS in this kernel.
    __syncthreads();
    if (tid < kGateBM && row < sel.doc) {
      const uint32_t key = order_key(gv);
      atomicAdd(&sel_sh.hist[key >> 21], 1u);
      __hip_atomic_store(&sel.ws[sel_keys_word(sel.doc) + row], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sel_publish_and_arrive<kGateThreads, true>(sel_sh, sel.ws)) return;
    // The ring is free: its three stages hold the keys while the last
    // workgroup ranks.
    constexpr int kPage = GateRing<H>::kPage;
    constexpr int kBlockTok = GateRing<H>::kBlockTok;
    SelKeys kp;
    kp.page[0] = reinterpret_cast<uint32_t*>(st0);
    kp.page[1] = reinterpret_cast<uint32_t*>(st1);
    kp.page[2] = reinterpret_cast<uint32_t*>(st2);
    kp.page_tokens = kPage;
    kp.block_tokens = kBlockTok;
    select_finish<kGateThreads>(sel_sh, kp, sel.doc, sel.kd, sel.ws);
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

template <bool SEL>
static hipError_t launch_gate_any(int64_t n, int d, int hidden, const void* h, int64_t ld_h, const void* w1,
                                  const float* b1, const float* w2, float b2, float* g, float* s, GateSel sel,
                                  hipStream_t stream) {
  if (!grid_fits((n + kGateBM - 1) / kGateBM, kGateThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n + kGateBM - 1) / kGateBM));
  const auto* hh = static_cast<const uint16_t*>(h);
  const auto* ww = static_cast<const uint16_t*>(w1);
  switch (hidden) {
    case 64:
      hipLaunchKernelGGL((gate_bf16_kernel<64, SEL>), grid, dim3(kGateThreads), 0, stream, hh, ld_h, (int)n, d, ww,
                         b1, w2, b2, g, s, sel);
      break;
    case 128:
      hipLaunchKernelGGL((gate_bf16_kernel<128, SEL>), grid, dim3(kGateThreads), 0, stream, hh, ld_h, (int)n, d,
                         ww, b1, w2, b2, g, s, sel);
      break;
    default:
      hipLaunchKernelGGL((gate_bf16_kernel<256, SEL>), grid, dim3(kGateThreads), 0, stream, hh, ld_h, (int)n, d,
                         ww, b1, w2, b2, g, s, sel);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_bf16(int64_t n, int d, int hidden, const void* h, int64_t ld_h,
                            const void* w1, const float* b1, const float* w2, float b2, float* g,
                            float* s, hipStream_t stream) {
  return launch_gate_any<false>(n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, GateSel{0, 0, nullptr}, stream);
}

int64_t gate_select_block_tokens(int hidden) {
  return hidden == 64 ? GateRing<64>::kBlockTok : (hidden == 128 ? GateRing<128>::kBlockTok : GateRing<256>::kBlockTok);
}

hipError_t launch_gate_select_bf16(int64_t n, int d, int hidden, const void* h, int64_t ld_h, const void* w1,
                                   const float* b1, const float* w2, float b2, float* g, float* s, int64_t k,
                                   int64_t q_len, int32_t* idx, void* workspace, void* h_out, float* g_out,
                                   int32_t* pos_out, hipStream_t stream) {
  const int64_t kept = k < n ? k : n;
  const GateSel sel{(int)(n - q_len), (int)(kept - q_len), static_cast<uint32_t*>(workspace)};
  hipError_t e = launch_gate_any<true>(n, d, hidden, h, ld_h, w1, b1, w2, b2, g, s, sel, stream);
  if (e != hipSuccess) return e;
  return launch_compact(g, n, k, q_len, idx, workspace, h, ld_h * 2, d * 2, h_out, g_out, pos_out, stream);
}

hipError_t launch_gate_f32(int64_t n, int d, int hidden, const float* h, int64_t ld_h,
                           const float* w1, const float* b1, const float* w2, float b2, float* g,
                           float* s, hipStream_t stream) {
  if (!grid_fits((n + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n + 3) / 4));
  hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(256), 0, stream, h, ld_h, (int)n, d, hidden, w1, b1,
                     w2, b2, g, s);
  return hipGetLastError();
}

}  // namespace tg
