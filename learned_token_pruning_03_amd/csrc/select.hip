// Stage 2 -- top-K selection with the question tail protected, on gfx950.
//
// TokenGate paper page (thelatestinai.com), Figure 1(a),(b): a top-K
// selector at layer L keeps K tokens; aitualizate.com article, section "3. Las
// capas superiores procesan únicamente los tokens seleccionados": only the
// document part may be pruned, the question always stays.  Tie and order
// rules (this library's reading): larger g first, ties to the lower index,
// NaN last, -0 == +0; output ascending with the tail last.
//
// One 1024-thread workgroup per prompt.  Scores become 32-bit keys whose
// unsigned order is the rank order.  Each thread owns KPT consecutive
// document tokens (held in registers when the prompt fits, re-read per pass
// otherwise).  The K-th largest key T is found by MSB-first radix passes of
// up to 11 bits, starting below the common prefix of the smallest and largest
// key, with a 2048-bin LDS histogram and a block suffix scan per pass.  A
// final block scan over (count > T, count == T) places every kept index at
// its ascending slot; the first `need` tokens equal to T (by index) are kept.
#include "select_core.h"

namespace tg {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kRadixBits = 11;
constexpr int kRadix = 1 << kRadixBits;

struct SelShared {
  uint32_t hist[kRadix];
  uint32_t red[kSelWaves][2];
  uint32_t bcast[4];
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Block-wide exclusive scan of two counters; returns the block totals.
__device__ __forceinline__ void block_excl_scan2(SelShared& sh, uint32_t a, uint32_t b, uint32_t& ea,
                                                 uint32_t& eb, uint32_t& ta, uint32_t& tb) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a, lane);
  const uint32_t ib = wave_incl_scan(b, lane);
  if (lane == 63) {
    sh.red[wave][0] = ia;
    sh.red[wave][1] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t xa = sh.red[w][0], xb = sh.red[w][1];
    if (w < wave) {
      pa += xa;
      pb += xb;
    }
    ta += xa;
    tb += xb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  __syncthreads();
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ g,
                                                            int n_single, int64_t k, int q_single,
                                                            const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ qlens,
                                                            int batch, int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cu_kept) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;

  // ---- this prompt's extent and its output offset -------------------------
  int64_t start = 0;
  int n = n_single;
  int q = q_single;
  int64_t off = 0;
  if (cu) {
    start = cu[b];
    n = cu[b + 1] - cu[b];
    q = qlens[b];
    // off = sum over earlier prompts of min(k, N_b'); block reduction.
    uint32_t part = 0;
    for (int bb = tid; bb < b; bb += kSelThreads) {
      const int64_t nb = cu[bb + 1] - cu[bb];
      part += (uint32_t)(nb < k ? nb : k);
    }
    uint32_t e0, e1, t0, t1;
    block_excl_scan2(sh, part, 0u, e0, e1, t0, t1);
    off = t0;
    if (b == 0) {
      // cu_kept[j] = sum_{b' < j} min(k, N_b')
      for (int j = tid; j <= batch; j += kSelThreads) {
        uint32_t acc = 0;
        for (int bb = 0; bb < j; ++bb) {
          const int64_t nb = cu[bb + 1] - cu[bb];
          acc += (uint32_t)(nb < k ? nb : k);
        }
        cu_kept[j] = (int32_t)acc;
      }
    }
  }
  const int kept = (int)(k < n ? k : n);
  int32_t* out = idx + off;
  if (n <= 0) return;
  if (q < 0 || q > kept) {  // invalid prompt: poison its slots
    for (int i = tid; i < kept; i += kSelThreads) out[i] = -1;
    return;
  }
  const int doc = n - q;
  const int kd = kept - q;
  if (kd >= doc) {  // budget covers the prompt: identity
    for (int i = tid; i < n; i += kSelThreads) out[i] = i;
    return;
  }
  for (int i = tid; i < q; i += kSelThreads) out[kd + i] = doc + i;  // protected tail
  if (kd == 0) return;

  // ---- keys ----------------------------------------------------------------
  constexpr int kChunk = kSelThreads * KPT;
  const int nchunks = (doc + kChunk - 1) / kChunk;
  const float* gs = g + start;
  const bool vec_ok = ((start & 3) == 0);
  uint32_t key[KPT];

  auto load_chunk = [&](int c) {
    const int base = c * kChunk + tid * KPT;
    if (vec_ok && base + KPT <= doc) {
#pragma unroll
      for (int j = 0; j < KPT; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(gs + base + j);
        key[j] = order_key(v[0]);
        key[j + 1] = order_key(v[1]);
        key[j + 2] = order_key(v[2]);
        key[j + 3] = order_key(v[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) key[j] = (base + j < doc) ? order_key(gs[base + j]) : 0u;
    }
  };
  auto nvalid = [&](int c) {
    const int base = c * kChunk + tid * KPT;
    const int r = doc - base;
    return r <= 0 ? 0 : (r >= KPT ? KPT : r);
  };

  if (nchunks == 1) load_chunk(0);

  // ---- pass 0: smallest and largest key ------------------------------------
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int c = 0; c < nchunks; ++c) {
    if (nchunks > 1) load_chunk(c);
    const int nv = nvalid(c);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < nv) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sh.red[wave][0] = kmin;
    sh.red[wave][1] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kmin = min(kmin, sh.red[w][0]);
    kmax = max(kmax, sh.red[w][1]);
  }
  __syncthreads();

  // ---- radix passes: find T = the kd-th largest key --------------------------
  const uint32_t diff = kmin ^ kmax;
  int known = diff ? __clz(diff) : 32;  // leading bits shared by every key
  uint32_t prefix = known == 0 ? 0u : (kmax >> (32 - known));
  uint32_t need = (uint32_t)kd;  // keys still to take at or below the prefix
  while (known < 32) {
    const int w = (32 - known) < kRadixBits ? (32 - known) : kRadixBits;
    const int shift = 32 - known - w;
    const uint32_t mask = (1u << w) - 1u;
    for (int i = tid; i < kRadix; i += kSelThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_chunk(c);
      const int nv = nvalid(c);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t kk = key[j];
        const bool match = (j < nv) && (known == 0 || (kk >> (32 - known)) == prefix);
        if (match) atomicAdd(&sh.hist[(kk >> shift) & mask], 1u);
      }
    }
    __syncthreads();
    // Suffix counts: thread t owns bins 2t, 2t+1; scan in descending bin order.
    if (tid == 0) {  // defaults, overwritten by exactly one thread below
      sh.bcast[0] = 0u;
      sh.bcast[1] = need;
    }
    const int rt = kSelThreads - 1 - tid;  // thread rt owns bins 2rt+1 (high), 2rt
    const uint32_t hi = sh.hist[2 * rt + 1], lo = sh.hist[2 * rt];
    uint32_t above, dummy, tot, tot2;
    // Exclusive scan in thread order == bins strictly above this pair.
    block_excl_scan2(sh, hi + lo, 0u, above, dummy, tot, tot2);
    if (above < need && above + hi >= need) {
      sh.bcast[0] = 2 * rt + 1;
      sh.bcast[1] = need - above;
    } else if (above + hi < need && above + hi + lo >= need) {
      sh.bcast[0] = 2 * rt;
      sh.bcast[1] = need - above - hi;
    }
    __syncthreads();
    prefix = (prefix << w) | sh.bcast[0];
    need = sh.bcast[1];
    known += w;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // ---- compaction in index order --------------------------------------------
  uint32_t run_gt = 0, run_eq = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (nchunks > 1) load_chunk(c);
    const int nv = nvalid(c);
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < nv) {
        cgt += key[j] > T;
        ceq += key[j] == T;
      }
    uint32_t egt, eeq, tgt, teq;
    block_excl_scan2(sh, cgt, ceq, egt, eeq, tgt, teq);
    uint32_t gt_before = run_gt + egt;
    uint32_t eq_before = run_eq + eeq;
    const int base = c * kChunk + tid * KPT;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (j < nv) {
        const uint32_t kk = key[j];
        if (kk > T) {
          const uint32_t slot = gt_before + min(eq_before, need);
          if (slot < (uint32_t)kd) out[slot] = base + j;
          ++gt_before;
        } else if (kk == T) {
          const uint32_t slot = gt_before + eq_before;
          if (eq_before < need && slot < (uint32_t)kd) out[slot] = base + j;
          ++eq_before;
        }
      }
    }
    run_gt += tgt;
    run_eq += teq;
  }
}

template <int KPT>
void launch_kpt(const float* g, int n, int64_t k, int q, const int32_t* cu, const int32_t* qlens,
                int batch, int32_t* idx, int32_t* cu_kept, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel<KPT>, dim3(batch), dim3(kSelThreads), 0, stream, g, n, k, q, cu,
                     qlens, batch, idx, cu_kept);
}

// ---- several workgroups per prompt ------------------------------------------
// The same selection with the top digit counted by ceil(doc / 4096)
// workgroups of 1024 threads (4 keys each) in LDS, then added to the
// workspace histogram with device atomics.  The last workgroup to arrive
// finishes the selection alone (select_finish): no grid-wide barrier and no
// waiting, so every workgroup runs to its end whatever the dispatch order.
constexpr int kHistThreads = 1024;
constexpr int kHistKpt = 4;
constexpr int kHistChunk = kHistThreads * kHistKpt;

__global__ __launch_bounds__(256) void sel_clear_kernel(uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kSelWsWords; i += 256) ws[i] = 0u;
}

template <int KPT_FIN>
__global__ __launch_bounds__(kHistThreads) void sel_hist_finish_kernel(const float* __restrict__ g, int doc, int kd,
                                                                       int q, int32_t* __restrict__ out,
                                                                       uint32_t* __restrict__ ws) {
  __shared__ SelFinishShared sh;
  for (int i = threadIdx.x; i < kSelBins; i += kHistThreads) sh.hist[i] = 0u;
  __syncthreads();
  const int base = blockIdx.x * kHistChunk + threadIdx.x * kHistKpt;
  if (base + kHistKpt <= doc && (reinterpret_cast<uintptr_t>(g) & 15u) == 0) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + base);
#pragma unroll
    for (int j = 0; j < kHistKpt; ++j) atomicAdd(&sh.hist[order_key(v[j]) >> 21], 1u);
  } else {
#pragma unroll
    for (int j = 0; j < kHistKpt; ++j)
      if (base + j < doc) atomicAdd(&sh.hist[order_key(g[base + j]) >> 21], 1u);
  }
  __syncthreads();
  if (!sel_publish_and_arrive<kHistThreads>(sh, ws)) return;
  select_finish<kHistThreads, KPT_FIN>(sh, g, doc, kd, q, out, ws);
}

}  // namespace

hipError_t launch_select(const float* g, int64_t n, int64_t k, int64_t q_len, const int32_t* cu_seqlens,
                         const int32_t* q_lens, int batch, int64_t max_seqlen, int32_t* idx,
                         int32_t* cu_kept, hipStream_t stream) {
  if (!grid_fits(batch, kSelThreads)) return hipErrorInvalidConfiguration;
  // Smallest register footprint that holds the longest prompt; longer
  // prompts stream their keys through the same registers once per pass.
  const int64_t m = max_seqlen;
  if (m <= kSelThreads * 4)
    launch_kpt<4>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  else if (m <= kSelThreads * 8)
    launch_kpt<8>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  else if (m <= kSelThreads * 16)
    launch_kpt<16>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  else if (m <= kSelThreads * 32)
    launch_kpt<32>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  else if (m <= kSelThreads * 64)
    launch_kpt<64>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  else
    launch_kpt<32>(g, (int)n, k, (int)q_len, cu_seqlens, q_lens, batch, idx, cu_kept, stream);
  return hipGetLastError();
}

int64_t select_mw_workspace_bytes(int64_t) { return kSelWsBytes; }

hipError_t launch_select_mw(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx, void* workspace,
                            bool ws_clean, hipStream_t stream) {
  const int64_t kept = k < n ? k : n;
  const int64_t doc = n - q_len, kd = kept - q_len;
  // Nothing to rank (budget covers the document, or only the tail is kept):
  // the one-workgroup kernel writes the identity or the tail.
  if (kd <= 0 || kd >= doc) return launch_select(g, n, k, q_len, nullptr, nullptr, 1, n, idx, nullptr, stream);
  const int64_t blocks = (doc + kHistChunk - 1) / kHistChunk;
  if (!grid_fits(blocks, kHistThreads)) return hipErrorInvalidConfiguration;
  auto* ws = static_cast<uint32_t*>(workspace);
  if (!ws_clean) hipLaunchKernelGGL(sel_clear_kernel, dim3(1), dim3(256), 0, stream, ws);
  hipLaunchKernelGGL(sel_hist_finish_kernel<32>, dim3((unsigned)blocks), dim3(kHistThreads), 0, stream, g, (int)doc,
                     (int)kd, (int)q_len, idx, ws);
  return hipGetLastError();
}

}  // namespace tg
