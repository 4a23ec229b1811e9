// Device pieces of the top-K selection shared by the selection kernels
// (select.hip) and the gate kernel that selects in its last workgroup
// (gate.hip).  Internal; not part of the public ABI.
//
// TokenGate paper page (thelatestinai.com), Figure 1(a),(b): a top-K selector
// at layer L keeps K tokens; aitualizate.com article, section "3. Las capas
// superiores procesan únicamente los tokens seleccionados": only the document
// may be pruned, the question always stays.  Order rules (this library's
// reading): larger g first, ties to the lower index, NaN last, -0 == +0;
// kept indices ascending with the question tail last.
//
// Workspace of the multi-workgroup forms (uint32 words, zero between calls):
//   [0, 2048)   counts of the top 11 bits (31..21) of every document key,
//               added by every workgroup with device atomics;
//   [2048]      arrival counter: the workgroup that brings it to gridDim.x is
//               the last one, sees every count and every score, and finishes
//               the selection alone.  It clears both before it returns.
#pragma once

#include "tg_internal.h"

namespace tg {

constexpr int kSelRadixBits = 11;
constexpr int kSelBins = 1 << kSelRadixBits;
constexpr int kSelWsCounter = kSelBins;         // word index of the arrival counter
constexpr int kSelWsWords = kSelBins + 64;      // 8448 bytes: histogram, counter, padding
constexpr int64_t kSelWsBytes = kSelWsWords * 4;

// Unsigned order of the key == rank order of the score: NaN -> 0 (lowest),
// -0 -> +0, negatives reversed below positives.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelFinishShared {
  uint32_t hist[kSelBins];
  uint32_t red[16][2];
  uint32_t bcast[4];
};

__device__ __forceinline__ uint32_t sel_wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Block-wide exclusive scan of two counters in thread order; also returns
// the block totals.  Ends with a barrier, so `red` can be reused at once.
template <int THREADS>
__device__ __forceinline__ void sel_block_scan2(SelFinishShared& sh, uint32_t a, uint32_t b, uint32_t& ea,
                                                uint32_t& eb, uint32_t& ta, uint32_t& tb) {
  constexpr int NW = THREADS / kWave;
  static_assert(NW <= 16, "block too large");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t ia = sel_wave_incl_scan(a, lane);
  const uint32_t ib = sel_wave_incl_scan(b, lane);
  if (lane == 63) {
    sh.red[wave][0] = ia;
    sh.red[wave][1] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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

// In sh.hist (kSelBins bins, counts of the keys still in play), the bin that
// holds the need-th largest key and how many keys of that bin are still to
// take.  Thread t owns kSelBins / THREADS consecutive bins, highest first.
template <int THREADS>
__device__ __forceinline__ void sel_resolve(SelFinishShared& sh, uint32_t need, uint32_t& bin, uint32_t& rest) {
  constexpr int PER = kSelBins / THREADS;
  static_assert(PER >= 1 && PER * THREADS == kSelBins, "bins per thread");
  const int top = kSelBins - 1 - (int)threadIdx.x * PER;
  uint32_t loc[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    loc[i] = sh.hist[top - i];
    sum += loc[i];
  }
  if (threadIdx.x == 0) {  // defaults, overwritten by exactly one thread below
    sh.bcast[0] = 0u;
    sh.bcast[1] = need;
  }
  uint32_t above, dummy, tot, tot2;
  sel_block_scan2<THREADS>(sh, sum, 0u, above, dummy, tot, tot2);
  if (above < need && above + sum >= need) {
    uint32_t cum = above;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum + loc[i] >= need) {
        sh.bcast[0] = (uint32_t)(top - i);
        sh.bcast[1] = need - cum;
        break;
      }
      cum += loc[i];
    }
  }
  __syncthreads();
  bin = sh.bcast[0];
  rest = sh.bcast[1];
  __syncthreads();
}

// Adds this workgroup's counts (sh.hist) to the workspace histogram, then
// counts the workgroup in.  Returns true in exactly one workgroup: the last
// to arrive, which then sees every count and every score written before the
// arrival of any workgroup.  Every thread of the block must call it.
template <int THREADS>
__device__ __forceinline__ bool sel_publish_and_arrive(SelFinishShared& sh, uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kSelBins; i += THREADS) {
    const uint32_t c = sh.hist[i];
    if (c) atomicAdd(&ws[i], c);
  }
  __threadfence();  // release: this thread's score stores and count atomics
  __syncthreads();
  if (threadIdx.x == 0) sh.bcast[2] = atomicAdd(&ws[kSelWsCounter], 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  const bool last = sh.bcast[2] != 0u;
  if (last) __threadfence();  // acquire: every other workgroup's stores and counts
  return last;
}

// The rest of the selection, in one workgroup of THREADS threads, once the
// workspace holds the top-digit histogram of all `doc` document keys of
// g[0, doc):
//   - the top digit's bin holding the kd-th largest key, from the histogram
//     (rebuilt here from the keys if its total is not `doc`);
//   - bits 20..10, then 9..0, of the keys still in play, counted in LDS: the
//     kd-th largest key T and `need`, how many keys equal to T are kept;
//   - one block scan over (count > T, count == T) places every kept index at
//     its ascending slot, the first `need` keys equal to T by index;
//   - the question tail [doc, doc + q) goes to slots [kd, kd + q).
// Requires 0 < kd < doc.  Clears the workspace histogram and counter.
// Each thread holds KPT consecutive keys of a THREADS * KPT chunk; a document
// of several chunks is re-read once per pass.
template <int THREADS, int KPT>
__device__ void select_finish(SelFinishShared& sh, const float* __restrict__ g, int doc, int kd, int q,
                              int32_t* __restrict__ out, uint32_t* __restrict__ ws) {
  const int tid = threadIdx.x;
  constexpr int kChunk = THREADS * KPT;
  const int nchunks = (doc + kChunk - 1) / kChunk;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(g) & 15u) == 0;
  uint32_t key[KPT];

  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int base = c * kChunk + tid * KPT;
    if (vec_ok && base + KPT <= doc) {
#pragma unroll
      for (int j = 0; j < KPT; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(g + base + j);
        key[j] = order_key(v[0]);
        key[j + 1] = order_key(v[1]);
        key[j + 2] = order_key(v[2]);
        key[j + 3] = order_key(v[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) key[j] = (base + j < doc) ? order_key(g[base + j]) : 0u;
    }
  };
  auto nvalid = [&](int c) __attribute__((always_inline)) {
    const int r = doc - (c * kChunk + tid * KPT);
    return r <= 0 ? 0 : (r >= KPT ? KPT : r);
  };

  // ---- top digit: the published histogram, moved to LDS; the workspace is
  // cleared for the next call as it is read.
  uint32_t part = 0;
  for (int i = tid; i < kSelBins; i += THREADS) {
    const uint32_t c = __hip_atomic_load(&ws[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.hist[i] = c;
    part += c;
    ws[i] = 0u;
  }
  if (tid == 0) ws[kSelWsCounter] = 0u;
  if (nchunks == 1) load_chunk(0);
  uint32_t e0, e1, total, t1;
  sel_block_scan2<THREADS>(sh, part, 0u, e0, e1, total, t1);
  if (total != (uint32_t)doc) {
    // Not the histogram of these keys (a workspace that was not left clean):
    // count the top digit here instead.
    for (int i = tid; i < kSelBins; i += THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_chunk(c);
      const int nv = nvalid(c);
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (j < nv) atomicAdd(&sh.hist[key[j] >> 21], 1u);
    }
    __syncthreads();
  }

  uint32_t prefix, need;
  sel_resolve<THREADS>(sh, (uint32_t)kd, prefix, need);

  // ---- bits 20..10, then 9..0, of the keys that share the prefix so far.
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int known = pass == 0 ? 11 : 22;
    const int w = pass == 0 ? 11 : 10;
    const int shift = 32 - known - w;
    const uint32_t mask = (1u << w) - 1u;
    for (int i = tid; i < kSelBins; i += THREADS) sh.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) load_chunk(c);
      const int nv = nvalid(c);
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t kk = key[j];
        if (j < nv && (kk >> (32 - known)) == prefix) atomicAdd(&sh.hist[(kk >> shift) & mask], 1u);
      }
    }
    __syncthreads();
    uint32_t bin, rest;
    sel_resolve<THREADS>(sh, need, bin, rest);
    prefix = (prefix << w) | bin;
    need = rest;
  }
  const uint32_t T = prefix;

  // ---- compaction in index order.
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
    sel_block_scan2<THREADS>(sh, cgt, ceq, egt, eeq, tgt, teq);
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
  for (int i = tid; i < q; i += THREADS) out[kd + i] = doc + i;  // protected tail
}

}  // namespace tg
