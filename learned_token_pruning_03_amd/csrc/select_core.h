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
// Workspace of the multi-workgroup forms (uint32 words):
//   [0, 2048)   counts of the top 11 bits (31..21) of every document key,
//               added by every workgroup with device atomics;
//   [2048]      arrival counter: the workgroup that brings it to gridDim.x is
//               the last one, sees every count and every score, and ranks
//               alone.  It clears the counts and the counter (zero between
//               calls) and writes the rest:
//   [2049]      T, the key of the kd-th largest document score;
//   [2050]      need, how many document keys equal to T are kept;
//   [2051]      the number of copy items (below);
//   [2112 + 2c] for each 64-token chunk c of the document: the number of its
//               keys above T, then equal to T, in the chunks before it (the
//               second written as 0 when need is 0: no equal key is kept);
//   then        copy items, chunk * 16 + part: part p of chunk c stands for
//               the chunk's kept tokens of rank 8p .. 8p + 7 (at most 8
//               rows per item, however the kept tokens cluster);
//   [sel_keys_word(doc)]  the order key of every document score, written by
//               the workgroup that counted it (past the L2), so that the
//               last workgroup copies them straight into LDS; padded to a
//               whole number of 256-key blocks.
// The kernels after it read T, need, the chunk counts and the items: one
// workgroup per chunk (indices only) or per item (indices and rows) places
// its kept tokens without any global scan.
#pragma once

#include "tg_internal.h"

namespace tg {

constexpr int kSelRadixBits = 11;
constexpr int kSelBins = 1 << kSelRadixBits;
constexpr int kSelWsCounter = kSelBins;  // word index of the arrival counter
constexpr int kSelWsT = kSelBins + 1;
constexpr int kSelWsNeed = kSelBins + 2;
constexpr int kSelWsItems = kSelBins + 3;    // number of copy items
constexpr int kSelWsChunks = kSelBins + 64;  // first chunk count
constexpr int kCompactChunk = 64;            // tokens per chunk
constexpr int kItemRows = 8;                 // kept rows per copy item

__host__ __device__ inline int64_t sel_chunks(int64_t n) { return (n + kCompactChunk - 1) / kCompactChunk; }
// Copy items of a prompt of n tokens, at most: sum over chunks of
// ceil(kept_c / 8) <= chunks + kept / 8.
__host__ __device__ inline int64_t sel_max_items(int64_t n) { return sel_chunks(n) + (n + kItemRows - 1) / kItemRows; }
__host__ __device__ inline int64_t sel_items_word(int64_t n) { return kSelWsChunks + 2 * sel_chunks(n); }
__host__ __device__ inline int64_t sel_keys_word(int64_t n) { return (sel_items_word(n) + sel_max_items(n) + 63) / 64 * 64; }
__host__ __device__ inline int64_t sel_keys_words(int64_t n) { return (n + 255) / 256 * 256; }
// Workspace bytes for a prompt of n tokens.
inline int64_t sel_ws_bytes(int64_t n) { return (sel_keys_word(n) + sel_keys_words(n)) * (int64_t)sizeof(uint32_t); }

// Unsigned order of the key == rank order of the score: NaN -> 0 (lowest),
// -0 -> +0, negatives reversed below positives.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelMaxBlockChunks = 512;  // 64-token chunks per block of keys held in LDS

struct alignas(16) SelFinishShared {
  uint32_t hist[kSelBins];  // filled by 16-byte global -> LDS copies: 16-byte aligned
  uint32_t sink[kWave];  // per-lane target of the counting atomics of keys not in play (never read)
  uint32_t red[16][2];
  uint32_t bcast[4];
};

// A block of keys held in LDS, in up to three pages (the gate keeps them in
// the three stages of its ring).  The 64-token chunk starting at token i of
// the block sits in page i / page_tokens.  block_tokens and page_tokens are
// multiples of 256 (the keys are copied in 256-key blocks); block_tokens is at
// most 64 * kSelMaxBlockChunks and 3 * page_tokens.
struct SelKeys {
  uint32_t* page[3];
  int page_tokens;
  int block_tokens;
};

// Selects between the three pages with constant indices: an index computed at
// run time would put the pointer array in scratch memory.
__device__ __forceinline__ uint32_t* sel_key_ptr(const SelKeys& k, int i) {
  if (i >= 2 * k.page_tokens) return k.page[2] + (i - 2 * k.page_tokens);
  if (i >= k.page_tokens) return k.page[1] + (i - k.page_tokens);
  return k.page[0] + i;
}

// Inclusive scan over the 64 lanes of a wave on the DPP lane network (row
// shifts within 16-lane rows, then the row broadcasts of lanes 15 and 31):
// six moves with no LDS round trip.
__device__ __forceinline__ uint32_t sel_wave_incl_scan(uint32_t v, int lane) {
  const int rl = lane & 15;
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  if (rl >= 1) v += t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  if (rl >= 2) v += t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  if (rl >= 4) v += t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  if (rl >= 8) v += t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x142, 0xf, 0xf, false);  // row_bcast:15
  if ((lane & 31) >= 16) v += t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x143, 0xf, 0xf, false);  // row_bcast:31
  if (lane >= 32) v += t;
  return v;
}

// Barrier for data exchanged through LDS only: each wave waits for its own
// LDS accesses, then meets the others.  __syncthreads would also wait for
// every global access in flight (key copies still landing, stores).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until at most n (0 <= n <= N) of this wave's memory operations are
// outstanding; n is the same for the whole wave.
template <int N>
__device__ __forceinline__ void wait_vm_n(int n) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (n >= N)
      wait_vm<N>();
    else
      wait_vm_n<N - 1>(n);
  }
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
  lds_barrier();
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
  lds_barrier();
}

// Block-wide exclusive scan of three counters with one LDS round trip; also
// returns the totals.
template <int THREADS>
__device__ __forceinline__ void sel_block_scan3(SelFinishShared& sh, const uint32_t (&v)[3], uint32_t (&ex)[3],
                                                uint32_t (&tot)[3]) {
  constexpr int NW = THREADS / kWave;
  static_assert(NW <= 8, "block too large for the three-counter scan");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t inc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) inc[c] = sel_wave_incl_scan(v[c], lane);
  if (lane == 63) {
#pragma unroll
    for (int c = 0; c < 3; ++c) (&sh.red[0][0])[3 * wave + c] = inc[c];
  }
  lds_barrier();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    uint32_t pre = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = (&sh.red[0][0])[3 * w + c];
      if (w < wave) pre += x;
      t += x;
    }
    ex[c] = pre + inc[c] - v[c];
    tot[c] = t;
  }
  lds_barrier();
}

// In sh.hist (kSelBins bins, counts of the keys still in play), the bin that
// holds the need-th largest key, how many keys of that bin are still to take
// (rest) and how many keys the bin holds (count).  Thread t owns
// kSelBins / THREADS consecutive bins, highest first.
// bin0_extra: counts in bin 0 that are not keys still in play (padding),
// taken out as the bins are read.
template <int THREADS>
__device__ __forceinline__ void sel_resolve(SelFinishShared& sh, uint32_t need, uint32_t& bin, uint32_t& rest,
                                            uint32_t& count, uint32_t* total = nullptr, uint32_t bin0_extra = 0u) {
  constexpr int PER = kSelBins / THREADS;
  static_assert(PER >= 1 && PER * THREADS == kSelBins, "bins per thread");
  const int top = kSelBins - 1 - (int)threadIdx.x * PER;
  uint32_t loc[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    loc[i] = sh.hist[top - i] - (top - i == 0 ? bin0_extra : 0u);
    sum += loc[i];
  }
  if (threadIdx.x == 0) {  // defaults, overwritten by exactly one thread below
    sh.bcast[0] = 0u;
    sh.bcast[1] = need;
    sh.bcast[3] = 0u;
  }
  uint32_t above, dummy, tot, tot2;
  sel_block_scan2<THREADS>(sh, sum, 0u, above, dummy, tot, tot2);
  if (total) *total = tot;
  if (above < need && above + sum >= need) {
    uint32_t cum = above;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum + loc[i] >= need) {
        sh.bcast[0] = (uint32_t)(top - i);
        sh.bcast[1] = need - cum;
        sh.bcast[3] = loc[i];
        break;
      }
      cum += loc[i];
    }
  }
  lds_barrier();
  bin = sh.bcast[0];
  rest = sh.bcast[1];
  count = sh.bcast[3];
  lds_barrier();
}

// Adds this workgroup's counts (sh.hist) to the workspace histogram, then
// counts the workgroup in.  Returns true in exactly one workgroup: the last
// to arrive.  Every thread of the block must call it.
//
// No agent-scope fence on the way: on this multi-XCD part such a fence writes
// back the whole L2 of the XCD, which costs microseconds per workgroup.
// Instead everything another workgroup will read is written past the L2
// (device atomics for the counts, agent-scope atomic stores for the keys),
// each thread waits until its own writes have completed (vmcnt 0) before the
// barrier, and only then does one thread count the workgroup in.  The last
// workgroup then drops its L2's copies (an agent-scope acquire: an
// invalidate, no write-back) before it reads the keys.
// ACQUIRE: the last workgroup reads data that other workgroups of the same
// kernel wrote; without it, only data from an earlier kernel.
template <int THREADS, bool ACQUIRE>
__device__ __forceinline__ bool sel_publish_and_arrive(SelFinishShared& sh, uint32_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kSelBins; i += THREADS) {
    const uint32_t c = sh.hist[i];
    if (c) atomicAdd(&ws[i], c);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) sh.bcast[2] = atomicAdd(&ws[kSelWsCounter], 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  const bool last = sh.bcast[2] != 0u;
  if (ACQUIRE && last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// The rest of the selection, in one workgroup of THREADS threads, once the
// workspace holds the top-digit histogram of all `doc` document keys and the
// keys themselves (at sel_keys_word(doc), written past the L2 by the
// workgroups that counted them):
//   - the top digit's bin holding the kd-th largest key, from the histogram
//     (rebuilt here from the keys if its total is not `doc`);
//   - bits 20..10, then 9..0, of the keys still in play, counted in LDS: the
//     kd-th largest key T and `need`, how many keys equal to T are kept.
//     When the bin a pass settles on is taken whole, every key at or above
//     that prefix is kept and the remaining passes are skipped;
//   - block scans give every 64-token chunk its counts before it and list
//     the copy items.
// Requires 0 < kd < doc.  Clears the workspace histogram and counter.
// Thread t owns chunk t of the block held in LDS (its 16 groups of 4 keys
// rotated by t, so that the 16 lanes of a quarter-wave read 16 different
// bank groups); a document of several blocks is re-read once per pass.  A
// single workgroup runs this once: each phase reads the thread's 64 keys into
// registers with all its LDS reads in flight, then works from the registers
// (a counting pass issues one LDS atomic per key: to its bin if the key is
// still in play, else to its lane's sink word).
// Chunks wholly past the document take no part; in the one chunk the
// document ends in, the keys past its end are set to 0 (the key of NaN) in
// registers, so no pass tests a key's index; wherever a pass counts key 0
// (histogram bin 0 of a prefix that is itself 0, or T == 0) those padding
// keys are taken back out.  Each histogram pass is compiled
// for its own digit (a phase known only at run time would make every key pay
// for both digit extractions and a select).
template <int THREADS>
__device__ __forceinline__ void select_finish(SelFinishShared& sh, const SelKeys& kp, int doc, int kd,
                                              uint32_t* __restrict__ ws) {
  constexpr int PER = kSelBins / THREADS;
  constexpr int kMaxIt = kSelMaxBlockChunks * kCompactChunk / (4 * THREADS);  // 16-byte loads per thread per block
  static_assert(PER * THREADS == kSelBins && kMaxIt >= 1 && THREADS >= kSelMaxBlockChunks, "block shape");
  static_assert(kMaxIt * (THREADS / kWave) * 256 == kSelMaxBlockChunks * kCompactChunk, "one copy per 256 keys");
  const int tid = threadIdx.x;
  const int B = kp.block_tokens;
  const int nblocks = (doc + B - 1) / B;
  const uint32_t* const keys = ws + sel_keys_word(doc);
  const bool owner = tid < B / kCompactChunk;  // this thread owns a chunk of every block
  uint32_t* const mine = sel_key_ptr(kp, owner ? tid * kCompactChunk : 0);
  auto slot_of = [](uint32_t* chunk, int t, int grp) __attribute__((always_inline)) {
    return chunk + 4 * ((grp + t) & 15);
  };

  // Keys of block c into LDS by global -> LDS copies (no register round
  // trip), all in flight at once after the barrier that lets the previous
  // block's readers finish.  A wave's copy moves a 256-key block (4 chunks);
  // lane l fills slot l % 16 of chunk l / 16, so it fetches the group of 4
  // keys that the chunk's rotation puts in that slot.  Blocks past the
  // document are not copied; keys past it in the last block are stale and
  // never counted (see read_chunk).
  // Valid keys of this thread's chunk in block c.
  auto nvalid = [&](int c) __attribute__((always_inline)) {
    const int r = owner ? doc - (c * B + tid * kCompactChunk) : 0;
    return r <= 0 ? 0 : (r >= kCompactChunk ? kCompactChunk : r);
  };
  int cur = -1;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Issues the copies of block c; returns how many this wave issued.
  auto issue_block = [&](int c) __attribute__((always_inline)) {
    const int base = c * B;
    const int cc = (tid & 63) >> 4, j = tid & 15;
    int issued = 0;
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
      const int wb = it * (THREADS / kWave) + wv;  // this wave's 256-key block
      const int i0 = wb * 256;
      if (i0 < B && base + i0 < doc) {
        const int t = 4 * wb + cc;  // the chunk (and owner thread) this lane's slot belongs to
        dma16(keys + base + i0 + cc * kCompactChunk + 4 * ((j - t) & 15),
              (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)sel_key_ptr(kp, i0));
        ++issued;
      }
    }
    return issued;
  };
  auto load_block = [&](int c) __attribute__((always_inline)) {
    __syncthreads();  // the previous block's readers are done
    issue_block(c);
    wait_vm<0>();
    __syncthreads();
    cur = c;
  };
  // Padding keys (value 0): the tail of the chunk the document ends in.
  const uint32_t pad_total = (uint32_t)((kCompactChunk - doc % kCompactChunk) % kCompactChunk);
  // All 64 keys of this thread's chunk (16 reads in flight), those past the
  // document's end set to 0 (only in the chunk the document ends in).
  auto read_chunk = [&](u32x4 (&k)[16], int nv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) k[i] = *reinterpret_cast<const u32x4*>(slot_of(mine, tid, i));
    if (nv < kCompactChunk) {
#pragma unroll
      for (int j = 0; j < 64; ++j) k[j >> 2][j & 3] = j < nv ? k[j >> 2][j & 3] : 0u;
    }
  };

  // ---- top digit: the published histogram and the first block of keys,
  // both by global -> LDS copies (the caller has dropped its L2's stale
  // lines), the histogram first: waiting for it leaves the keys in flight
  // while the top digit is resolved below.
  static_assert(kSelBins * 4 == THREADS * 16, "one 16-byte copy of the histogram per thread");
  dma16(ws + 4 * tid, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)&sh.hist[0] + wv * 1024);
  wait_vm_n<kMaxIt>(issue_block(0));
  lds_barrier();

  // Phases over the blocks of keys, the current block kept in LDS between
  // phases: 0 counts the top digit again (only if the published counts do
  // not add up to doc: a workspace that was not left clean), 1 and 2 count
  // bits 20..10 and 9..0 of the keys that share the prefix found so far,
  // 3 counts the keys above and equal to T per chunk and lists the items.
  uint32_t prefix = 0, need = (uint32_t)kd, T = 0;
  int phase = 1;
  {
    uint32_t bin, rest, cnt, total;
    sel_resolve<THREADS>(sh, need, bin, rest, cnt, &total);
    if (total != (uint32_t)doc) {
      phase = 0;
    } else {
      prefix = bin;
      need = rest;
      if (rest == cnt) {  // the bin is taken whole: keys > T are those with top digit >= prefix
        T = (prefix << 21) - 1u;
        need = 0u;
        phase = 3;
      }
    }
  }
  // The first block's keys.
  wait_vm<0>();
  __syncthreads();
  cur = 0;
  uint32_t* items = ws + sel_items_word(doc);
  uint32_t run_gt = 0, run_eq = 0, run_items = 0;
#pragma unroll 1
  for (; phase < 4; ++phase) {
    if (phase < 3) {
      for (int i = tid; i < kSelBins; i += THREADS) sh.hist[i] = 0u;
      lds_barrier();
    }
#pragma unroll 1
    for (int c = 0; c < nblocks; ++c) {
      if (c != cur) load_block(c);
      const int nv = nvalid(c);
      const bool live = nv > 0;  // owns a chunk with document tokens in this block
      u32x4 k[16];
      if (live) read_chunk(k, nv);
      if (phase < 3) {
        // One LDS atomic per key, straight from the registers, for every key:
        // a key not in play adds to its lane's sink word instead of a bin.  A
        // predicated atomic would put a chain of exec-mask updates around
        // every key, which the keys cannot overlap; a loop over the live keys
        // alone would run as many rounds as the fullest chunk of the wave
        // holds (kept tokens cluster, so one chunk can hold many).
        uint32_t* const sink = &sh.sink[tid & (kWave - 1)];
        auto pass = [&](auto ph) __attribute__((always_inline)) {
          constexpr int P = decltype(ph)::value;
#pragma unroll
          for (int j = 0; j < 64; ++j) {
            const uint32_t kk = k[j >> 2][j & 3];
            if constexpr (P == 0) {
              atomicAdd(&sh.hist[kk >> 21], 1u);
            } else if constexpr (P == 1) {
              atomicAdd((kk >> 21) == prefix ? &sh.hist[(kk >> 10) & 2047u] : sink, 1u);
            } else {
              atomicAdd((kk >> 10) == prefix ? &sh.hist[kk & 1023u] : sink, 1u);
            }
          }
        };
        if (live) {
          if (phase == 1)
            pass(std::integral_constant<int, 1>{});
          else if (phase == 2)
            pass(std::integral_constant<int, 2>{});
          else
            pass(std::integral_constant<int, 0>{});
        }
        continue;
      }
      // phase 3: counts of this chunk, then block scans in chunk order.  With
      // need == 0 no key equal to T is kept, and those counts are not needed
      // (they are written as 0).
      uint32_t cgt = 0, ceq = 0;
      if (live) {
        if (need == 0u) {
#pragma unroll
          for (int j = 0; j < 64; ++j) cgt += k[j >> 2][j & 3] > T ? 1u : 0u;
        } else {
#pragma unroll
          for (int j = 0; j < 64; ++j) {
            const uint32_t kk = k[j >> 2][j & 3];
            cgt += kk > T ? 1u : 0u;
            ceq += kk == T ? 1u : 0u;
          }
          if (T == 0u) ceq -= (uint32_t)(kCompactChunk - nv);  // the padding keys
        }
      }
      uint32_t gt_b, eq_b, tgt, teq, eni, tni, ni;
      if (need == 0u) {  // keys equal to T are never kept: the items follow from cgt alone
        ni = nv > 0 ? (cgt + kItemRows - 1) / kItemRows : 0u;
        const uint32_t v3[3] = {cgt, ceq, ni};
        uint32_t ex3[3], tot3[3];
        sel_block_scan3<THREADS>(sh, v3, ex3, tot3);
        gt_b = run_gt + ex3[0];
        eq_b = run_eq + ex3[1];
        eni = ex3[2];
        tgt = tot3[0];
        teq = tot3[1];
        tni = tot3[2];
      } else {
        uint32_t egt, eeq;
        sel_block_scan2<THREADS>(sh, cgt, ceq, egt, eeq, tgt, teq);
        gt_b = run_gt + egt;
        eq_b = run_eq + eeq;
        const uint32_t kept = cgt + (min(eq_b + ceq, need) - min(eq_b, need));
        ni = nv > 0 ? (kept + kItemRows - 1) / kItemRows : 0u;
        uint32_t dummy, tdummy;
        sel_block_scan2<THREADS>(sh, ni, 0u, eni, dummy, tni, tdummy);
      }
      if (nv > 0) {
        const int ch = c * (B / kCompactChunk) + tid;
        ws[kSelWsChunks + 2 * ch] = gt_b;
        ws[kSelWsChunks + 2 * ch + 1] = eq_b;
#pragma unroll 1
        for (uint32_t r = 0; r < ni; ++r) items[run_items + eni + r] = (uint32_t)ch * 16u + r;
      }
      run_gt += tgt;
      run_eq += teq;
      run_items += tni;
    }
    if (phase < 3) {
      lds_barrier();
      // The padding keys (0) were counted when this pass's prefix is 0: all
      // of them in digit 0.
      const bool pad_counted = phase == 0 || prefix == 0u;
      uint32_t bin, rest, cnt;
      sel_resolve<THREADS>(sh, need, bin, rest, cnt, nullptr, pad_counted ? pad_total : 0u);
      const int w = phase == 1 ? 11 : 10;
      const int bits_left = phase == 0 ? 21 : (phase == 1 ? 10 : 0);
      prefix = phase == 0 ? bin : (prefix << w) | bin;
      need = rest;
      if (phase == 2) {
        T = prefix;
      } else if (rest == cnt) {  // the bin is taken whole
        T = (prefix << bits_left) - 1u;
        need = 0u;
        phase = 2;  // next: phase 3
      }
    }
  }
  if (tid == 0) {
    ws[kSelWsT] = T;
    ws[kSelWsNeed] = need;
    ws[kSelWsItems] = run_items;
  }
  // ---- the counts and the counter are zero again for the next call.
#pragma unroll
  for (int i = 0; i < PER; ++i)
    __hip_atomic_store(&ws[tid + i * THREADS], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(&ws[kSelWsCounter], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tg
