// Upper-layer dense work on the kept tokens, on gfx950.
//
// aitualizate.com article, section "3. Las capas superiores procesan
// únicamente los tokens seleccionados": every layer above the selection layer
// runs on the K kept tokens only, so its projections and MLP are products of
// a [K, d] activation with the layer's weights.  The layer shape is the base
// model of the TokenGate paper page's setup table (Qwen3-1.7B, bf16): bias-free
// QKV and O projections and a SwiGLU MLP.  The LoRA adapters of that setup are
// taken as merged into the weights, so each projection is one plain product.
//
// One kernel, C = A W^T with A [M, Kin] and W [N, Kin] (nn.Linear layout, both
// Kin-contiguous), fp32 accumulation on v_mfma_f32_32x32x16_bf16, and three
// epilogues:
//   plain     C = bf16(A W^T)
//   residual  C = bf16(A W^T + R)               (R may alias C)
//   swiglu    C = bf16(SiLU(A Wg^T) * (A Wu^T))  (Wg, Wu [F, Kin]; C [M, F])
// A workgroup (4 waves, one per SIMD) owns a BM x 256 block of the product:
// BM rows of A against 256 rows of W (for swiglu: 128 rows of Wg and the
// matching 128 rows of Wu, so each output needs no exchange between waves).
// Each wave holds a (BM/2) x 128 accumulator tile (256 fp32 registers per lane
// at BM = 256, which the compiler keeps in the accumulation registers).
// A and W stream through a four-stage LDS ring of 32-wide k-chunks filled by
// global_load_lds (compiler-blind, so in-flight copies are never drained by
// the compiler's wait-count pass); three chunks are in flight while the
// matrix cores work on the fourth.  Fragments of the next chunk's first half
// are read between the two halves of the current chunk's MFMAs, so after the
// one barrier per chunk the matrix pipe restarts on data already in registers.
#include <type_traits>

#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kGemmThreads = 256;  // 4 waves: 2 along M x 2 along N
constexpr int kGemmBN = 256;       // rows of W per workgroup
constexpr int kGemmBK = 32;        // k elements per ring stage (64 bytes of a row)
constexpr int kGemmStages = 4;

enum { kEpiPlain = 0, kEpiResidual = 1, kEpiSwiglu = 2 };

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* w;   // [N, Kin], or Wg [F, Kin] for swiglu
  const uint16_t* w2;  // Wu [F, Kin] for swiglu
  const uint16_t* r;   // residual [M, N]
  uint16_t* c;   // output columns [0, s1)
  uint16_t* c1;  // output columns [s1, s2) (plain epilogue; s1 = s2 = n when unused)
  uint16_t* c2;  // output columns [s2, n)
  int64_t lda, ldw, ldr, ldc, ld1, ld2;
  int s1, s2;
  int m, n, k;  // n = output columns (F for swiglu)
  int tiles_m, tiles_n;
};

// LDS rows are 64 bytes = 4 chunks of 16 bytes.  Chunk c of row r sits at
// slot c ^ ((r >> 2) & 3): the 16 rows read by each quarter of a
// ds_read_b128 then cover all 64 banks once.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <int BM, int EPI>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int MT = BM / 64;                          // 32-row tiles per wave
  constexpr int NT = 4;                                // 32-column tiles per wave
  constexpr int A_BYTES = BM * 64;
  constexpr int STAGE = A_BYTES + kGemmBN * 64;
  constexpr int A_DMA = BM * 4 / kGemmThreads;         // 16-byte copies per lane per chunk (A)
  constexpr int B_DMA = kGemmBN * 4 / kGemmThreads;    // same for W
  constexpr int PER = A_DMA + B_DMA;                   // vmcnt increments per chunk
  static_assert(PER <= 16 && 2 * PER < 64, "wait counts");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kGemmStages * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, r32 = lane & 31;

  // Workgroup -> tile.  Consecutive workgroups go to different XCDs (round
  // robin), so first give each XCD a contiguous range of the linear order,
  // then walk that order in groups of 4 tile rows: the tiles an XCD runs at
  // once share 4 row panels of A and a few column panels of W in its L2.
  int lin = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
  constexpr int GM = 4;
  const int group = lin / (GM * p.tiles_n);
  const int first = group * GM;
  const int gsize = min(p.tiles_m - first, GM);
  const int tm = first + (lin % (GM * p.tiles_n)) % gsize;
  const int tn = (lin % (GM * p.tiles_n)) / gsize;
  const int m0 = tm * BM;
  const int n0 = tn * (EPI == kEpiSwiglu ? kGemmBN / 2 : kGemmBN);

  // Copy q of a chunk: 64 lanes fill one 1 KB block = 16 rows x 4 slots; lane
  // l lands at row 16 b + l/4, slot l%4, which holds chunk (l%4) ^ ((row>>2)&3).
  const uint8_t* src[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const bool isA = q < A_DMA;
    const int blk = (isA ? q : q - A_DMA) * 4 + wave;
    const int row = blk * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const uint16_t* base;
    if (isA) {
      const int gr = min(m0 + row, p.m - 1);  // rows past M read a valid row; results dropped
      base = p.a + (int64_t)gr * p.lda;
    } else if (EPI == kEpiSwiglu) {
      base = row < kGemmBN / 2 ? p.w + (int64_t)(n0 + row) * p.ldw : p.w2 + (int64_t)(n0 + row - kGemmBN / 2) * p.ldw;
    } else {
      base = p.w + (int64_t)(n0 + row) * p.ldw;
    }
    src[q] = reinterpret_cast<const uint8_t*>(base) + chunk * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  auto issue_one = [&](int q, int kt) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + (kt & (kGemmStages - 1)) * STAGE;
    const int blk = (q < A_DMA ? q : q - A_DMA) * 4 + wave;
    dma16(src[q] + kt * (kGemmBK * 2), sb + (q < A_DMA ? 0 : A_BYTES) + blk * 1024);
  };

  // Fragment rows: A tiles of this wave, and the W tiles (for swiglu, tiles 0-1
  // are gate rows and 2-3 the matching up rows).
  auto wrow = [&](int j) __attribute__((always_inline)) {
    if (EPI == kEpiSwiglu) return (j < 2 ? 0 : kGemmBN / 2) + wn * 64 + (j & 1) * 32 + r32;
    return wn * 128 + j * 32 + r32;
  };
  auto read_frags = [&](int kt, int u, bf16x8* af, bf16x8* bfr) __attribute__((always_inline)) {
    const uint8_t* sb = ring + (kt & (kGemmStages - 1)) * STAGE;
    const int chunk = u * 2 + half;
#pragma unroll
    for (int i = 0; i < MT; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(sb + swz(wm * (BM / 2) + i * 32 + r32, chunk));
#pragma unroll
    for (int j = 0; j < NT; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sb + A_BYTES + swz(wrow(j), chunk));
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // MFMAs of one 16-wide half-chunk; copies of chunk kt_next (if any) go out
  // spread between them.
  auto mfmas = [&](const bf16x8* af, const bf16x8* bfr, int kt_next) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        constexpr int EVERY = (MT * NT) / PER;  // >= 1
        const int mi = i * NT + j;
        if (kt_next >= 0 && mi % EVERY == EVERY - 1 && mi / EVERY < PER) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one(mi / EVERY, kt_next);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };

  const int nk = p.k / kGemmBK;
  for (int c = 0; c < 3 && c < nk; ++c)
#pragma unroll
    for (int q = 0; q < PER; ++q) issue_one(q, c);
  if (nk >= 3)
    wait_vm<2 * PER>();
  else if (nk == 2)
    wait_vm<PER>();
  else
    wait_vm<0>();
  plain_barrier();

  bf16x8 a0[MT], b0[NT], a1[MT], b1[NT];
  // One chunk: read the second half's fragments, run the first half's MFMAs
  // (with the copies of chunk kt+3 when there is one), wait until chunk kt+1
  // has landed (MODE 2: two chunks may stay in flight, 1: one, 0: none) and
  // every wave is done with chunk kt (whose stage the next step's copies
  // overwrite), read the next chunk's first-half fragments, then run the
  // second half's MFMAs.  MODE -1: last chunk, no next.  The loop is peeled
  // by mode so that each copy of the body has no branches.
  auto step = [&](int kt, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    read_frags(kt, 1, a1, b1);
    mfmas(a0, b0, MODE == 2 ? kt + 3 : -1);
    if constexpr (MODE >= 0) {
      if constexpr (MODE == 2)
        wait_vm<2 * PER>();
      else if constexpr (MODE == 1)
        wait_vm<PER>();
      else
        wait_vm<0>();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of chunk kt are done
      plain_barrier();
      read_frags(kt + 1, 0, a0, b0);
    }
    mfmas(a1, b1, -1);
  };
  using M2 = std::integral_constant<int, 2>;
  using M1 = std::integral_constant<int, 1>;
  using M0 = std::integral_constant<int, 0>;
  using ML = std::integral_constant<int, -1>;

  read_frags(0, 0, a0, b0);
  int kt = 0;
  for (; kt + 3 < nk; ++kt) step(kt, M2{});
  if (kt + 2 < nk) step(kt++, M1{});
  if (kt + 1 < nk) step(kt++, M0{});
  step(kt, ML{});

  // ---- epilogue.  acc[i][j][e] holds row wm*BM/2 + i*32 + 8*(e/4) + 4*half +
  // e%4 of the tile and column (W row) wrow(j).  A 256-column tile lies in one
  // of the (up to) three output ranges; pick its buffer once.
  uint16_t* cbase = p.c;
  int64_t ldo = p.ldc;
  int c0 = 0;
  if (EPI == kEpiPlain && n0 >= p.s2) {
    cbase = p.c2;
    ldo = p.ld2;
    c0 = p.s2;
  } else if (EPI == kEpiPlain && n0 >= p.s1) {
    cbase = p.c1;
    ldo = p.ld1;
    c0 = p.s1;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
      if (row >= p.m) continue;
      uint16_t* crow = cbase + (int64_t)row * ldo;
      if (EPI == kEpiSwiglu) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float gv = acc[i][j][e], uv = acc[i][j + 2][e];
          // SiLU(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal.
          const float sg = gv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv * kLog2e));
          const int col = n0 + wn * 64 + j * 32 + r32;
          reinterpret_cast<__bf16*>(crow)[col] = (__bf16)(sg * uv);
        }
      } else {
        const uint16_t* rrow = EPI == kEpiResidual ? p.r + (int64_t)row * p.ldr : nullptr;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int col = n0 + wn * 128 + j * 32 + r32;
          float v = acc[i][j][e];
          if (EPI == kEpiResidual) v += bf16_bits_to_f32(rrow[col]);
          reinterpret_cast<__bf16*>(crow)[col - c0] = (__bf16)v;
        }
      }
    }
  }
}

template <int BM, int EPI>
hipError_t launch_bm(GemmArgs p, hipStream_t stream) {
  p.tiles_m = (int)(((int64_t)p.m + BM - 1) / BM);
  p.tiles_n = p.n / (EPI == kEpiSwiglu ? kGemmBN / 2 : kGemmBN);
  if (!grid_fits((int64_t)p.tiles_m * p.tiles_n, kGemmThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI>), dim3(p.tiles_m * p.tiles_n), dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& p, hipStream_t stream) {
  // 256-row tiles when they still give a full chip (>= 256 workgroups),
  // else 128-row tiles.
  const int64_t cols = EPI == kEpiSwiglu ? kGemmBN / 2 : kGemmBN;
  const int64_t big = ((p.m + 255) / 256) * (p.n / cols);
  return big >= 256 ? launch_bm<256, EPI>(p, stream) : launch_bm<128, EPI>(p, stream);
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, const void* w,
                            const void* w2, int64_t ldw, const void* r, int64_t ldr, void* c, int64_t ldc,
                            hipStream_t stream) {
  return launch_gemm_bf16_split(epi, m, n, k, a, lda, w, w2, ldw, r, ldr, c, ldc, nullptr, 0, n, nullptr, 0, n,
                                stream);
}

hipError_t launch_gemm_bf16_split(int epi, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                                  const void* w, const void* w2, int64_t ldw, const void* r, int64_t ldr, void* c,
                                  int64_t ldc, void* c1, int64_t ld1, int64_t s1, void* c2, int64_t ld2, int64_t s2,
                                  hipStream_t stream) {
  GemmArgs p;
  p.c1 = static_cast<uint16_t*>(c1);
  p.c2 = static_cast<uint16_t*>(c2);
  p.ld1 = ld1;
  p.ld2 = ld2;
  p.s1 = (int)s1;
  p.s2 = (int)s2;
  p.a = static_cast<const uint16_t*>(a);
  p.w = static_cast<const uint16_t*>(w);
  p.w2 = static_cast<const uint16_t*>(w2);
  p.r = static_cast<const uint16_t*>(r);
  p.c = static_cast<uint16_t*>(c);
  p.lda = lda;
  p.ldw = ldw;
  p.ldr = ldr;
  p.ldc = ldc;
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  switch (epi) {
    case kEpiPlain: return launch_epi<kEpiPlain>(p, stream);
    case kEpiResidual: return launch_epi<kEpiResidual>(p, stream);
    case kEpiSwiglu: return launch_epi<kEpiSwiglu>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tg
