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
//
// Also here: the multi-workgroup forms of the same selection (up to 32768
// document tokens: a histogram kernel whose last workgroup ranks, then a
// compaction; longer documents: six short kernels), and the compaction that
// also copies the kept rows, used after the gate that ranks in its last
// workgroup.
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
// Up to one LDS block of document keys (kFinishBlock), the same selection in
// three short kernels with no grid-wide barrier:
//   sel_clear_kernel        zeroes the workspace's histogram and counter;
//   sel_hist_finish_kernel  ceil(doc / 4096) workgroups of 512 threads count
//                           the top 11 bits of 8 keys per thread in LDS, add
//                           them to the workspace and store the keys there;
//                           the last workgroup to arrive copies the keys into
//                           LDS and ranks alone (select_finish): T, need and
//                           the counts before every 64-token chunk;
//   compact_kernel          one workgroup per 64-token chunk writes the kept
//                           indices of its chunk.
// No workgroup ever waits for another, whatever the dispatch order.
constexpr int kHistThreads = 512;
constexpr int kHistKpt = 8;
constexpr int kHistChunk = kHistThreads * kHistKpt;

__global__ __launch_bounds__(256) void sel_clear_kernel(uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i <= kSelWsCounter; i += 256) ws[i] = 0u;
}

constexpr int kFinishBlock = kSelMaxBlockChunks * kCompactChunk;  // keys the last workgroup holds in LDS

__global__ __launch_bounds__(kHistThreads) void sel_hist_finish_kernel(const float* __restrict__ g, int doc, int kd,
                                                                       uint32_t* __restrict__ ws) {
  __shared__ SelFinishShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t keys[kFinishBlock];
  for (int i = threadIdx.x; i < kSelBins; i += kHistThreads) sh.hist[i] = 0u;
  __syncthreads();
  // Each key is counted and also stored in the workspace, past the L2: the
  // last workgroup copies the keys into LDS in this kernel.
  uint32_t* const wkeys = ws + sel_keys_word(doc);
  const int base = blockIdx.x * kHistChunk + threadIdx.x * kHistKpt;
  uint32_t key[kHistKpt];
  if (base + kHistKpt <= doc && (reinterpret_cast<uintptr_t>(g) & 15u) == 0) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(g + base);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(g + base + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      key[j] = order_key(v0[j]);
      key[4 + j] = order_key(v1[j]);
    }
#pragma unroll
    for (int j = 0; j < kHistKpt; ++j) {
      atomicAdd(&sh.hist[key[j] >> 21], 1u);
      __hip_atomic_store(&wkeys[base + j], key[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kHistKpt; ++j)
      if (base + j < doc) {
        const uint32_t kj = order_key(g[base + j]);
        atomicAdd(&sh.hist[kj >> 21], 1u);
        __hip_atomic_store(&wkeys[base + j], kj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  __syncthreads();
  if (!sel_publish_and_arrive<kHistThreads, true>(sh, ws)) return;
  SelKeys kp;
  kp.page[0] = kp.page[1] = kp.page[2] = keys;
  kp.page_tokens = kFinishBlock;
  kp.block_tokens = kFinishBlock;
  select_finish<kHistThreads>(sh, kp, doc, kd, ws);
}

// Where each kept token goes, from T, need and the chunk counts:
//   document token j (key k_j):  kept iff k_j > T, or k_j == T and fewer
//     than `need` keys equal to T come before it; its slot is the number of
//     kept document tokens before it;
//   question token j >= doc:     always kept, slot kd + (j - doc).
struct CompactArgs {
  const float* g;
  int n, doc, kd, q;
  const uint32_t* ws;
  int32_t* idx;
  const uint8_t* h;   // rows of h (gather_items_kernel)
  int64_t ld_bytes;   // bytes between rows of h
  int row_chunks;     // 16-byte pieces per row
  uint8_t* h_out;     // [kept, row_chunks * 16] contiguous
  float* g_out;       // or NULL
  int32_t* pos_out;   // or NULL
  int tail_items;     // ceil(q / 8)
};

// Decision for the 64 tokens of chunk c, one per lane of a wave: the token,
// its score, whether it is kept and its slot.
struct ChunkLane {
  int j;
  float gj;
  bool kept;
  int slot;
};

// T and need are the ranking's threshold key and the count of tokens equal to
// it to keep (passed in, so callers can load them early).
__device__ __forceinline__ ChunkLane decide_chunk(const CompactArgs& a, int c, int lane, uint32_t T, uint32_t need) {
  ChunkLane r;
  r.j = c * kCompactChunk + lane;
  const bool in_doc = r.j < a.doc;
  const bool in_tail = !in_doc && r.j < a.n;
  r.gj = (r.j < a.n) ? a.g[r.j] : 0.0f;
  const uint32_t key = order_key(r.gj);
  uint32_t gt_b = 0, eq_b = 0;
  if (c * kCompactChunk < a.doc) {
    gt_b = a.ws[kSelWsChunks + 2 * c];
    eq_b = a.ws[kSelWsChunks + 2 * c + 1];
  }
  const bool gt = in_doc && key > T;
  const bool eq = in_doc && key == T;
  const uint64_t bg = __ballot(gt), be = __ballot(eq);
  const uint32_t pg = __builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0u));
  const uint32_t pe = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
  const uint32_t eq_rank = eq_b + pe;
  const uint32_t doc_slot = gt_b + pg + min(eq_rank, need);
  r.slot = in_doc ? (int)doc_slot : a.kd + (r.j - a.doc);
  // A slot outside [0, kd) only comes from a workspace that does not hold
  // this call's counts: nothing is written for it (compared unsigned, so
  // counts that wrap past 2^31 cannot give a negative slot either).
  r.kept = in_tail || ((gt || (eq && eq_rank < need)) && doc_slot < (uint32_t)a.kd);
  return r;
}

// Indices only: one wave per 64-token chunk of [0, n).
__global__ __launch_bounds__(64) void compact_kernel(CompactArgs a) {
  const ChunkLane r = decide_chunk(a, blockIdx.x, threadIdx.x, a.ws[kSelWsT], a.ws[kSelWsNeed]);
  if (r.kept) a.idx[r.slot] = r.j;
}

// Indices, rows, gate values and positions: one workgroup of 256 threads per
// item of at most 8 kept rows.  Workgroups [0, tail_items) take 8 question
// tokens each; the next ones take the items the ranking listed (those past
// the listed count return at once).  Wave 0 decides the item's chunk, then
// the four waves copy two rows each, both rows' loads in flight before the
// stores.
__global__ __launch_bounds__(256) void gather_items_kernel(CompactArgs a) {
  __shared__ int32_t s_src[kItemRows], s_slot[kItemRows];
  __shared__ float s_g[kItemRows];
  __shared__ int s_cnt;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  if (b < a.tail_items) {
    if (threadIdx.x < kItemRows) {
      const int i = b * kItemRows + threadIdx.x;
      if (i < a.q) {
        const int j = a.doc + i, slot = a.kd + i;
        a.idx[slot] = j;
        s_src[threadIdx.x] = j;
        s_slot[threadIdx.x] = slot;
        s_g[threadIdx.x] = a.g[j];
      }
      if (threadIdx.x == 0) s_cnt = min(kItemRows, a.q - b * kItemRows);
    }
  } else {
    const int item = b - a.tail_items;
    // The item count, this item's code and the threshold are loaded together
    // rather than one after another: the grid has sel_max_items(doc) item
    // workgroups, so the code slot lies in the workspace for each of them
    // (the code of an item past the count is never used).
    const uint32_t count = a.ws[kSelWsItems];
    const uint32_t code = a.ws[sel_items_word(a.doc) + item];
    const uint32_t T = a.ws[kSelWsT], need = a.ws[kSelWsNeed];
    if (item >= (int)count) return;
    // A chunk past the document only comes from a workspace that does not
    // hold this call's item list: nothing is read or written for it.
    if ((code >> 4) >= (uint32_t)sel_chunks(a.doc)) return;
    const int c = (int)(code >> 4), part = (int)(code & 15u);
    if (wave == 0) {
      const ChunkLane r = decide_chunk(a, c, lane, T, need);
      const uint64_t bk = __ballot(r.kept);
      const int kr = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bk, 0u));
      const int lo = part * kItemRows;
      if (r.kept && kr >= lo && kr < lo + kItemRows) {
        a.idx[r.slot] = r.j;
        s_src[kr - lo] = r.j;
        s_slot[kr - lo] = r.slot;
        s_g[kr - lo] = r.gj;
      }
      if (lane == 0) s_cnt = max(0, min(kItemRows, __popcll(bk) - lo));
    }
  }
  __syncthreads();
  const int nk = s_cnt;
  const int r0 = 2 * wave;
  const int nr = min(2, nk - r0);
  if (nr > 0) {
    for (int c0 = 0; c0 < a.row_chunks; c0 += 4 * kWave) {
      u32x4 v[2][4];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c0 + u * kWave + lane;
          if (rr < nr && cc < a.row_chunks)
            v[rr][u] = *reinterpret_cast<const u32x4*>(a.h + (int64_t)s_src[r0 + rr] * a.ld_bytes + cc * 16);
        }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c0 + u * kWave + lane;
          if (rr < nr && cc < a.row_chunks)
            *reinterpret_cast<u32x4*>(a.h_out + (int64_t)s_slot[r0 + rr] * a.row_chunks * 16 + cc * 16) = v[rr][u];
        }
    }
  }
  if (threadIdx.x < nk) {
    if (a.g_out) a.g_out[s_slot[threadIdx.x]] = s_g[threadIdx.x];
    if (a.pos_out) a.pos_out[s_slot[threadIdx.x]] = s_src[threadIdx.x];
  }
}

// ---- long documents: six kernels -------------------------------------------
// Above one LDS block of keys (kFinishBlock), one workgroup would re-read the
// scores block by block in every pass; there the same selection runs spread
// over ceil(doc / 2048) workgroups of 256 threads, one 2048-key chunk each, in
// six short kernels with no grid-wide barrier:
//   zero    clears the three histograms in the workspace;
//   hist<0> histograms bits [31:21] of every key (LDS, then device atomics);
//   hist<1> finds the bin holding the kd-th largest key from histogram 0 and
//           histograms bits [20:10] of the keys in that bin;
//   hist<2> the same one level down, bits [9:0];
//   count   resolves T and `need` from histogram 2 and counts, per chunk, the
//           keys above T and equal to T;
//   write   places every kept index at its ascending slot: the chunk's offset
//           is the sum of the counts of the chunks before it.
// Every workgroup resolves the previous histogram itself (the same scan, the
// same answer); workgroup 0 also stores the answer for the next kernel, each
// pass in its own slot, so that no kernel reads a slot it writes.  The
// workspace words these kernels use overlap the ones the fused and one-block
// forms expect to find zero (their histogram and arrival counter, words
// 0 .. kSelWsCounter): `write` zeroes them again on its way out, in
// workgroup 0, which reads none of them.
constexpr int kMwThreads = 256;
constexpr int kMwWaves = kMwThreads / kWave;
constexpr int kMwKpt = 8;
constexpr int kMwChunk = kMwThreads * kMwKpt;
constexpr int kMwH0 = 0, kMwH1 = 2048, kMwH2 = 4096;  // histogram offsets (uint32 words)
constexpr int kMwState = 5120;                        // per pass: (prefix, need) at kMwState + 2 * pass
constexpr int kMwCnt = 5128;                          // per chunk: (count > T, count == T)
constexpr int64_t kSelectMwMaxDoc = int64_t(1) << 24;  // each workgroup sums at most 8191 chunk counts
// The public workspace size (sel_ws_bytes) covers this layout for every
// document above kFinishBlock: at the smallest such document it holds 7748
// words against 5162 needed, and it grows by ~0.17 words per token against
// 0.001 here.
static_assert(kSelWsChunks + 3 * ((kFinishBlock + 1 + 63) / 64) + (kFinishBlock + 1 + 7) / 8 >=
                  kMwCnt + 2 * ((kFinishBlock + 1 + kMwChunk - 1) / kMwChunk),
              "workspace too small for the six-kernel form");

struct MwShared {
  uint32_t hist[2048];
  uint32_t red[kMwWaves][2];
  uint32_t bcast[2];
};

__device__ __forceinline__ void mw_excl_scan2(MwShared& sh, uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                              uint32_t& ta, uint32_t& tb) {
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
  for (int w = 0; w < kMwWaves; ++w) {
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

// This thread's keys (chunk blockIdx.x, KPT consecutive tokens per thread)
// and how many of them lie inside the document.
__device__ __forceinline__ int mw_load(const float* __restrict__ g, int doc, bool vec_ok, uint32_t (&key)[kMwKpt]) {
  const int base = blockIdx.x * kMwChunk + threadIdx.x * kMwKpt;
  const int nv = doc - base <= 0 ? 0 : (doc - base >= kMwKpt ? kMwKpt : doc - base);
  if (vec_ok && nv == kMwKpt) {
#pragma unroll
    for (int j = 0; j < kMwKpt; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(g + base + j);
      key[j] = order_key(v[0]);
      key[j + 1] = order_key(v[1]);
      key[j + 2] = order_key(v[2]);
      key[j + 3] = order_key(v[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMwKpt; ++j) key[j] = j < nv ? order_key(g[base + j]) : 0u;
  }
  return nv;
}

// Bin of an NB-bin histogram that holds the need-th largest counted key, and
// how many keys of that bin are still to take.  Thread t owns NB/256
// consecutive bins, highest first.
template <int NB>
__device__ __forceinline__ void mw_resolve(MwShared& sh, const uint32_t* __restrict__ h, uint32_t need,
                                           uint32_t& bin, uint32_t& rest) {
  constexpr int PER = NB / kMwThreads;
  const int top = NB - 1 - (int)threadIdx.x * PER;
  uint32_t loc[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    loc[i] = h[top - i];
    sum += loc[i];
  }
  if (threadIdx.x == 0) {  // defaults, overwritten by exactly one thread below
    sh.bcast[0] = 0u;
    sh.bcast[1] = need;
  }
  uint32_t above, dummy, tot, tot2;
  mw_excl_scan2(sh, sum, 0u, above, dummy, tot, tot2);
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

__global__ __launch_bounds__(kMwThreads) void mw_zero_kernel(uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kMwState; i += kMwThreads) ws[i] = 0u;
}

// PASS 0: bits [31:21] of every key; PASS 1: bits [20:10] of the keys whose
// top 11 bits equal the pass-0 bin; PASS 2: bits [9:0] below the 22-bit prefix.
template <int PASS>
__global__ __launch_bounds__(kMwThreads) void mw_hist_kernel(const float* __restrict__ g, int doc, int kd,
                                                             bool vec_ok, uint32_t* __restrict__ ws) {
  __shared__ MwShared sh;
  constexpr int NB = PASS == 2 ? 1024 : 2048;
  constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  uint32_t key[kMwKpt];
  const int nv = mw_load(g, doc, vec_ok, key);
  uint32_t prefix = 0;
  if (PASS > 0) {
    const uint32_t prev_prefix = PASS == 1 ? 0u : ws[kMwState + 0];
    const uint32_t prev_need = PASS == 1 ? (uint32_t)kd : ws[kMwState + 1];
    uint32_t bin, rest;
    mw_resolve<2048>(sh, ws + (PASS == 1 ? kMwH0 : kMwH1), prev_need, bin, rest);
    prefix = (prev_prefix << 11) | bin;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      ws[kMwState + 2 * (PASS - 1)] = prefix;
      ws[kMwState + 2 * (PASS - 1) + 1] = rest;
    }
  }
  for (int i = threadIdx.x; i < NB; i += kMwThreads) sh.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMwKpt; ++j) {
    const uint32_t kk = key[j];
    const bool match = j < nv && (PASS == 0 || (kk >> (SHIFT + (PASS == 2 ? 10 : 11))) == prefix);
    if (match) atomicAdd(&sh.hist[(kk >> SHIFT) & (NB - 1)], 1u);
  }
  __syncthreads();
  uint32_t* h = ws + (PASS == 0 ? kMwH0 : (PASS == 1 ? kMwH1 : kMwH2));
  for (int i = threadIdx.x; i < NB; i += kMwThreads) {
    const uint32_t c = sh.hist[i];
    if (c) atomicAdd(&h[i], c);
  }
}

// Resolves T (the kd-th largest document key) and `need` (how many keys equal
// to T are kept); stores them (workgroup 0) and this chunk's two counts.
__global__ __launch_bounds__(kMwThreads) void mw_count_kernel(const float* __restrict__ g, int doc, bool vec_ok,
                                                              uint32_t* __restrict__ ws) {
  __shared__ MwShared sh;
  uint32_t key[kMwKpt];
  const int nv = mw_load(g, doc, vec_ok, key);
  uint32_t bin, rest;
  mw_resolve<1024>(sh, ws + kMwH2, ws[kMwState + 3], bin, rest);
  const uint32_t T = (ws[kMwState + 2] << 10) | bin;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws[kMwState + 4] = T;
    ws[kMwState + 5] = rest;
  }
  uint32_t cgt = 0, ceq = 0;
#pragma unroll
  for (int j = 0; j < kMwKpt; ++j)
    if (j < nv) {
      cgt += key[j] > T;
      ceq += key[j] == T;
    }
  uint32_t egt, eeq, tgt, teq;
  mw_excl_scan2(sh, cgt, ceq, egt, eeq, tgt, teq);
  if (threadIdx.x == 0) {
    ws[kMwCnt + 2 * blockIdx.x] = tgt;
    ws[kMwCnt + 2 * blockIdx.x + 1] = teq;
  }
}

__global__ __launch_bounds__(kMwThreads) void mw_write_kernel(const float* __restrict__ g, int doc, int kd, int q,
                                                              bool vec_ok, const uint32_t* __restrict__ ws,
                                                              uint32_t* __restrict__ ws_clear,
                                                              int32_t* __restrict__ out) {
  __shared__ MwShared sh;
  uint32_t key[kMwKpt];
  const int nv = mw_load(g, doc, vec_ok, key);
  const uint32_t T = ws[kMwState + 4];
  const uint32_t need = ws[kMwState + 5];
  // This chunk's offset: the counts of every chunk before it.
  uint32_t pgt = 0, peq = 0;
  for (int c = threadIdx.x; c < (int)blockIdx.x; c += kMwThreads) {
    pgt += ws[kMwCnt + 2 * c];
    peq += ws[kMwCnt + 2 * c + 1];
  }
  uint32_t e0, e1, chunk_gt, chunk_eq;
  mw_excl_scan2(sh, pgt, peq, e0, e1, chunk_gt, chunk_eq);
  uint32_t cgt = 0, ceq = 0;
#pragma unroll
  for (int j = 0; j < kMwKpt; ++j)
    if (j < nv) {
      cgt += key[j] > T;
      ceq += key[j] == T;
    }
  uint32_t egt, eeq, tgt, teq;
  mw_excl_scan2(sh, cgt, ceq, egt, eeq, tgt, teq);
  uint32_t gt_before = chunk_gt + egt;
  uint32_t eq_before = chunk_eq + eeq;
  const int base = blockIdx.x * kMwChunk + threadIdx.x * kMwKpt;
#pragma unroll
  for (int j = 0; j < kMwKpt; ++j) {
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
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < q; i += kMwThreads) out[kd + i] = doc + i;  // protected tail
    for (int i = threadIdx.x; i <= kSelWsCounter; i += kMwThreads) ws_clear[i] = 0u;
  }
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

int64_t select_mw_workspace_bytes(int64_t n) { return sel_ws_bytes(n); }

hipError_t launch_compact(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx, const void* workspace,
                          const void* h, int64_t ld_h_bytes, int row_bytes, void* h_out, float* g_out,
                          int32_t* pos_out, hipStream_t stream) {
  const int64_t kept = k < n ? k : n;
  CompactArgs a;
  a.g = g;
  a.n = (int)n;
  a.doc = (int)(n - q_len);
  a.kd = (int)(kept - q_len);
  a.q = (int)q_len;
  a.ws = static_cast<const uint32_t*>(workspace);
  a.idx = idx;
  a.h = static_cast<const uint8_t*>(h);
  a.ld_bytes = ld_h_bytes;
  a.row_chunks = row_bytes / 16;
  a.h_out = static_cast<uint8_t*>(h_out);
  a.g_out = g_out;
  a.pos_out = pos_out;
  a.tail_items = (int)((q_len + kItemRows - 1) / kItemRows);
  if (h_out) {
    const int64_t blocks = a.tail_items + sel_max_items(a.doc);
    if (!grid_fits(blocks, 256)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gather_items_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  } else {
    const int64_t blocks = sel_chunks(n);
    if (!grid_fits(blocks, kWave)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(kWave), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_select_mw(const float* g, int64_t n, int64_t k, int64_t q_len, int32_t* idx, void* workspace,
                            bool ws_clean, hipStream_t stream) {
  const int64_t kept = k < n ? k : n;
  const int64_t doc = n - q_len, kd = kept - q_len;
  // Nothing to rank (budget covers the document, or only the tail is kept):
  // the one-workgroup kernel writes the identity or the tail.
  if (kd <= 0 || kd >= doc) return launch_select(g, n, k, q_len, nullptr, nullptr, 1, n, idx, nullptr, stream);
  auto* ws = static_cast<uint32_t*>(workspace);
  if (doc > kFinishBlock) {
    // More chunks than the per-chunk offset sums of the six-kernel form are
    // sized for: one workgroup does it.
    if (doc > kSelectMwMaxDoc) return launch_select(g, n, k, q_len, nullptr, nullptr, 1, n, idx, nullptr, stream);
    const int64_t chunks = (doc + kMwChunk - 1) / kMwChunk;
    if (!grid_fits(chunks, kMwThreads)) return hipErrorInvalidConfiguration;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(g) & 15u) == 0;
    const dim3 grid((unsigned)chunks);
    hipLaunchKernelGGL(mw_zero_kernel, dim3(1), dim3(kMwThreads), 0, stream, ws);
    hipLaunchKernelGGL(mw_hist_kernel<0>, grid, dim3(kMwThreads), 0, stream, g, (int)doc, (int)kd, vec_ok, ws);
    hipLaunchKernelGGL(mw_hist_kernel<1>, grid, dim3(kMwThreads), 0, stream, g, (int)doc, (int)kd, vec_ok, ws);
    hipLaunchKernelGGL(mw_hist_kernel<2>, grid, dim3(kMwThreads), 0, stream, g, (int)doc, (int)kd, vec_ok, ws);
    hipLaunchKernelGGL(mw_count_kernel, grid, dim3(kMwThreads), 0, stream, g, (int)doc, vec_ok, ws);
    hipLaunchKernelGGL(mw_write_kernel, grid, dim3(kMwThreads), 0, stream, g, (int)doc, (int)kd, (int)q_len, vec_ok,
                       ws, ws, idx);
    return hipGetLastError();
  }
  const int64_t blocks = (doc + kHistChunk - 1) / kHistChunk;
  if (!grid_fits(blocks, kHistThreads)) return hipErrorInvalidConfiguration;
  if (!ws_clean) hipLaunchKernelGGL(sel_clear_kernel, dim3(1), dim3(256), 0, stream, ws);
  hipLaunchKernelGGL(sel_hist_finish_kernel, dim3((unsigned)blocks), dim3(kHistThreads), 0, stream, g, (int)doc,
                     (int)kd, ws);
  return launch_compact(g, n, k, q_len, idx, ws, nullptr, 0, 0, nullptr, nullptr, nullptr, stream);
}

}  // namespace tg
