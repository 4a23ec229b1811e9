// Stage 4 -- token-gated causal GQA attention over the kept tokens, gfx950.
//
// TokenGate paper page (thelatestinai.com), Figure 1(c): every attention
// weight is multiplied by the gate value g_j of its key (and the weights
// renormalised); the page's Abstract and the aitualizate.com article, section
// "Cómo consigue entrenar una selección top-K": the importance score is a
// bias on the attention logits.  Both give softmax_j(scale*q.k_j + ln g_j).
// In base 2 with c = scale*log2 e:  t_ij = c * (q_i.k_j + log2 max(g_j, FLT_MIN) / c),
// p_ij = 2^(t_ij - m_i).  The bias term, divided by c, seeds the QK^T
// accumulator, so it enters the logit inside the MFMA and then takes part in
// the running maximum and the running sum like any other part of the logit.
//
// One bf16 kernel, attn_bf16_pp_kernel, in two forms: the gate bias of every
// visible key in one LDS table when it fits (8192 keys at head dim 128, 16384
// at 64, and always without a gate), else streamed tile by tile.
//
// One workgroup = 512 threads = 8 waves, two per SIMD:
//  * the two 4-wave groups split each query tile's key range (group 0 takes
//    the even 64-key tiles, group 1 the odd ones) and merge their partial
//    (max, sum, output) through LDS at the end of the tile;
//  * inside a group each wave owns 32 queries.  S^T = K Q^T runs on
//    v_mfma_f32_32x32x16_bf16 with Q held in registers as the B operand, so
//    each lane owns one query: its row max, row sum and rescale factor are
//    per-lane scalars, and P^T leaves the accumulators directly as the B
//    operand of O^T = V^T P^T (no LDS round trip for P);
//  * K and V tiles go from global memory straight into LDS (global_load_lds,
//    XOR-swizzled 256-byte rows); the V^T operand is read with
//    ds_read_b64_tr_b16, the transposing LDS read, so V needs no
//    transposition pass;
//  * the Q tile arrives the same way (into a V buffer not yet in use) and
//    the normalised output tile leaves through LDS as whole rows, so no load
//    or store instruction touches 32 query rows at once;
//  * the causal test runs only on tiles reaching past a wave's first query;
//  * the online softmax takes row maxima only on a wave's first tile; later
//    tiles reuse that reference maximum until a tile's weight sum shows a
//    weight above 2^64 (or overflow); that tile is redone against its row
//    maxima, and the wave then takes them on every tile, moving its
//    reference only when a logit exceeds it by more than 8 (log2 units);
//  * blockIdx -> (KV head, query head) puts all query heads of one KV head on
//    the same XCD, where they share that head's K/V in L2.
//  * a workgroup owns a pair of query tiles, (T-1-p) then p, so every
//    workgroup has the same causal work;
//  * the two groups alternate MFMA and VALU slots so that the two waves of a
//    SIMD overlap matrix and vector work, with copies issued three slots
//    ahead (see the kernel's own comment).
#include <cmath>

#include "tg_internal.h"

namespace tg {
namespace {

struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* g;          // gate values, or NULL: no gate (every key weighs 1)
  const float* head_gain;  // [hq] multiplier of the gate bias, or NULL: 1
  const int32_t* pos;
  uint8_t* o;
  float* lse;
  const int32_t* cu;
  int total;
  int hq;
  int hkv;
  float scale_log2;
};

template <int DH>
struct AttnCfg {
  static constexpr int BM = 128;                 // queries per tile (4 waves x 32)
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int CPR = DH / 8;             // 16-byte chunks per K/V row
  static constexpr int ROW = DH * 2;             // LDS bytes per K or V row (XOR-swizzled chunks)
  static constexpr int K_BYTES = BN * ROW;
  static constexpr int DMA = BN * CPR / 256;     // 16-byte direct loads per thread per tensor
  static constexpr int MD = DH / 32;             // 32-row blocks of O^T
  // The merge hands over half of each wave's O^T (MD/2 blocks of 16 fp32 per
  // lane, 4 waves) through one K buffer pair.
  static_assert(4 * (MD / 2) * 16 * 64 * 4 <= 2 * K_BYTES, "merge scratch (O) must fit in one buffer pair");
  // Chunk c of row r is stored at chunk c ^ swz(r).  K rows are read by
  // ds_read_b128 (16 consecutive rows, one chunk), V rows by the transposing
  // read (4 consecutive rows x 4 consecutive chunks per half-wave).
  static __device__ __forceinline__ int swz_k(int r) { return DH == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return DH == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 ping-pong kernel.
//
// 8 waves; group g takes the key tiles kt = 2t + g, and the two waves on each
// SIMD (one per group) never run the same kind of work at the same time.  Work is cut into
// slots separated by workgroup barriers.  Each group alternates
//   MFMA slot t:  O^T += V^T P^T for its tile t-1, then S^T = K Q^T for tile t
//   VALU slot t:  online softmax of tile t (P^T for the next MFMA slot)
// and group 1 runs one slot behind group 0, so in every slot one wave of each
// SIMD feeds the matrix core while the other runs the exp/max/sum VALU work.
// K and V have their own double buffers: K(t+2) and V(t+1) are copied in at
// the start of VALU slot t, three slots before they are read.  The gate bias
// comes from LDS (a table built once per tile pair, or a ring the copies
// feed), so the pipelined region holds no register loads from global memory.  Keys are
// visible when their kept index is at most the query's: with strictly
// increasing positions (the contract of the entry point) that is the same
// test as comparing positions.
template <int DH>
struct PPCfg {
  static constexpr int MAXK = DH == 128 ? 8192 : 16384;  // keys whose bias fits in LDS
};

// STREAM = false: the bias of every key the workgroup can see sits in one LDS
// table, built once per tile pair (prompts up to MAXK keys, or no gate).
// STREAM = true: wave 0 of each group copies the raw gate values of the
// group's key tile t+3 together with the other copies of batch t and, inside
// MFMA slot t, turns those of tile t+1 into its bias in a two-slot LDS ring:
// any prompt length, at a few percent more per tile.
template <int DH, bool STREAM>
__global__ __launch_bounds__(512) void attn_bf16_pp_kernel(AttnArgs a) {
  using C = AttnCfg<DH>;
  constexpr int KB = C::K_BYTES;  // one group's K (or V) tile
  constexpr int MAXK = PPCfg<DH>::MAXK;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t k_s0[2 * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t k_s1[2 * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_s0[2 * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_s1[2 * KB];
  __shared__ __attribute__((aligned(16))) float bias_all[STREAM ? 1 : MAXK];
  __shared__ __attribute__((aligned(16))) float graw[2][STREAM ? 4 : 1][BN];    // per group, 4 tile slots
  __shared__ __attribute__((aligned(16))) float bias_s[2][STREAM ? 2 : 1][BN];  // per group, 2 tile slots

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int w4 = wave & 3;
  const int gtid = tid & 255;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // Two 128-query tiles per workgroup: workgroup p takes tile T-1-p, then
  // tile p, so every workgroup does the same causal work (T tiles of keys).
  // rr = blockIdx % hq runs over the KV heads first, so all query heads of a
  // KV head land on one XCD and share its K/V in L2.
  const int hq = a.hq, hkv = a.hkv, group = hq / hkv;
  const int rr = blockIdx.x % hq;
  const int kvh = rr % hkv;
  const int head = kvh * group + rr / hkv;
  int64_t s0 = 0;
  int L = a.total;
  if (a.cu) {
    s0 = a.cu[blockIdx.y];
    L = a.cu[blockIdx.y + 1] - (int)s0;
  }
  const int ntiles = (L + C::BM - 1) / C::BM;
  // The short tile's keys are a prefix of the long tile's, so the bias table
  // built for the long tile serves both.  The tile body is a lambda called
  // twice rather than a loop: a loop keeps its values live across the back
  // edge and spills.
  const int pair = (int)(blockIdx.x / hq);
  auto tile_body = [&](const int mt, const bool pass0) __attribute__((always_inline)) {
  const int pass = pass0 ? 0 : 1;

  const uint8_t* kbase = a.k + ((s0 * hkv + kvh) * DH) * 2;
  const uint8_t* vbase = a.v + ((s0 * hkv + kvh) * DH) * 2;
  const uint32_t kvs = (uint32_t)((int64_t)hkv * DH * 2);  // bytes between consecutive keys
  const float c = a.scale_log2;
  const bool has_gate = a.g != nullptr;
  // Read before any copy is in flight: a register load waited for later would
  // also wait for the copies.
  const float gain = a.head_gain ? a.head_gain[head] : 1.0f;

  const int row0 = mt * C::BM;
  const int qi = row0 + w4 * 32 + r32;
  const int kend = min(L, row0 + C::BM);
  const int n_kt = (kend + BN - 1) / BN;
  const int niter = grp == 0 ? (n_kt + 1) / 2 : n_kt / 2;  // this group's tiles, kt = 2t + grp
  const int niter0 = (n_kt + 1) / 2;                        // group 0 has at least as many

  // Copy i of this thread fills chunk P = i*256 + gtid of a tile: row
  // r = P / CPR = i*(256/CPR) + gtid/CPR, stored slot gtid % CPR, holding
  // logical chunk slot ^ swz(r).  Both swizzles depend only on bits of r that
  // i does not touch.  The byte offset of copy i from the tile's first key is
  // fixed per lane; the tile's own offset kt*BN*kvs goes into the scalar base.
  // K/V bytes of one head span less than 2^31 (checked by the host).
  const int dma_r0 = gtid / C::CPR;
  uint32_t off_k[C::DMA], off_v[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const uint32_t rb = (uint32_t)(i * (256 / C::CPR) + dma_r0) * kvs;
    off_k[i] = rb + (uint32_t)(((gtid % C::CPR) ^ C::swz_k(dma_r0)) * 16);
    off_v[i] = rb + (uint32_t)(((gtid % C::CPR) ^ C::swz_v(dma_r0)) * 16);
  }
  auto lds_addr = [](uint8_t* ptr) __attribute__((always_inline)) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ptr;
  };
  const uint32_t k_addr[2] = {lds_addr(k_s0) + grp * KB, lds_addr(k_s1) + grp * KB};
  const uint32_t v_addr[2] = {lds_addr(v_s0) + grp * KB, lds_addr(v_s1) + grp * KB};
  auto issue = [&](const uint8_t* base, const uint32_t* off, int kt, uint32_t dst) __attribute__((always_inline)) {
    const uint8_t* tb = base + (size_t)((uint32_t)(kt * BN) * kvs);
    if ((kt + 1) * BN <= L) {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) dma16_sv(tb, off[i], dst + (i * 256 + w4 * 64) * 16);
    } else {  // last, partial tile: rows past the prompt re-read its last key
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        const int r = kt * BN + i * (256 / C::CPR) + dma_r0;
        const uint32_t o = off[i] - (uint32_t)(max(r - (L - 1), 0)) * kvs;
        dma16_sv(tb, o, dst + (i * 256 + w4 * 64) * 16);
      }
    }
  };

  // STREAM: raw gate values of this group's tile t (keys (2t + grp) * BN..)
  // into slot t % 4 by wave 0 of the group, lanes past the prompt re-reading
  // its last key; the bias of tile t from them, by the same wave (so its own
  // copy wait covers the data), into slot t % 2.
  const float inv_c = gain / c;  // gate bias times the head's gain
  const bool g_wave = STREAM && w4 == 0;
  auto issue_g = [&](int t) __attribute__((always_inline)) {
    if (g_wave) dma4(a.g + s0 + min((2 * t + grp) * BN + lane, L - 1),
                     lds_addr(reinterpret_cast<uint8_t*>(&graw[grp][t & 3][0])));
  };
  // The input is clamped to a normal number, where the hardware log2 is what
  // log2f computes.
  auto bias_of = [&](int t, float gj) __attribute__((always_inline)) {
    return (2 * t + grp) * BN + lane >= L ? -INFINITY : __builtin_amdgcn_logf(fmaxf(gj, kFltMin)) * inv_c;
  };
  auto g_count = [&](int t) __attribute__((always_inline)) { return (g_wave && t < niter) ? 1 : 0; };

  // ---- prologue: the Q tile and the gate values first, then the first K/V
  // copies, so that one wait covers Q and g while the copies keep landing.
  // The Q tile goes into the second V buffer (not written before the first
  // VALU slot) by global -> LDS copies of whole rows, laid out like a K tile:
  // loaded into registers directly, every load instruction would touch 32
  // query rows.  Copy i of this thread fills 16-byte slot P = 512 i + tid:
  // row P / CPR, holding logical chunk (P % CPR) ^ swz_k(row); rows past the
  // prompt re-read its last row.
  static_assert(C::BM * C::CPR % 512 == 0 && C::BM * C::ROW <= 2 * KB, "Q tile copies");
#pragma unroll
  for (int i = 0; i < C::BM * C::CPR / 512; ++i) {
    const int P = i * 512 + tid;
    const int r = P / C::CPR;
    const int src_row = min(row0 + r, L - 1);
    dma16(a.q + (((s0 + src_row) * hq + head) * DH) * 2 + ((P % C::CPR) ^ C::swz_k(r)) * 16,
          lds_addr(v_s1) + (i * 512 + wave * 64) * 16);
  }
  // Bias table, in units of the raw score (log2 g / c), for every key this
  // query tile can see (rounded up to whole key tiles); keys past the prompt
  // get -inf.
  const int nb = n_kt * BN;
  constexpr int GPT = STREAM ? 1 : (MAXK + 511) / 512;
  float gv[GPT];
  // Unconditional loads at a clamped index: a predicated load would let the
  // compiler sink each log2 into its own branch and wait for every load in turn.
  // Without a gate these loads read the position array instead (same length,
  // values unused): a NULL test inside the loop would split the loads into
  // branches that each wait for their own load.
  const float* gsrc = has_gate ? a.g + s0 : reinterpret_cast<const float*>(a.pos + s0);
  if (!STREAM && pass == 0) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) gv[i] = gsrc[min(tid + 512 * i, L - 1)];
  }
  // Copies per wave in batch b: K of tile b+2, V of tile b+1 (and, STREAM,
  // the gate values of tile b+3); here go the gate values of tile 0, batch
  // -2 (K(0), g(1)) and batch -1 (K(1), V(0), g(2)).
  if (0 < niter) issue_g(0);
  if (0 < niter) issue(kbase, off_k, grp, k_addr[0]);
  if (1 < niter) issue_g(1);
  if (1 < niter) issue(kbase, off_k, 2 + grp, k_addr[1]);
  if (0 < niter) issue(vbase, off_v, grp, v_addr[0]);
  if (2 < niter) issue_g(2);
  {
    // Q, g and the gate values of tile 0 have landed once at most the two
    // batches are outstanding; the copies may not have.
    const int nc = (0 < niter ? 2 * C::DMA : 0) + (1 < niter ? C::DMA : 0) + g_count(1) + g_count(2);
    if (nc == 3 * C::DMA + 2)
      wait_vm<3 * C::DMA + 2>();
    else if (nc == 3 * C::DMA + 1)
      wait_vm<3 * C::DMA + 1>();
    else if (nc == 3 * C::DMA)
      wait_vm<3 * C::DMA>();
    else if (nc == 2 * C::DMA)
      wait_vm<2 * C::DMA>();
    else
      wait_vm<0>();
  }
  if (g_wave && 0 < niter) bias_s[grp][0][lane] = bias_of(0, graw[grp][0][lane]);
  if (!STREAM && pass == 0 && !has_gate && tid < BN) bias_all[tid] = 0.0f;
  if (!STREAM && pass == 0 && a.g) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int j = tid + 512 * i;
      if (j < nb) bias_all[j] = j < L ? log2f(fmaxf(gv[i], kFltMin)) * inv_c : -INFINITY;
    }
  }
  const int G = lane >> 4, ia = (lane >> 2) & 3, ib = lane & 3;
  // K fragment offset of k-step ks is koff0 ^ (ks << 5) and the V^T offset of
  // 32-row block md is voff0 ^ (md << 6): the swizzle XOR and the step land
  // in disjoint bits, for both head sizes.
  const uint32_t koff0 = r32 * C::ROW + ((half ^ C::swz_k(r32)) * 16);
  const int vrow = 4 * (G >> 1) + ia;
  const uint32_t voff0 = vrow * C::ROW + (((2 * (G & 1) + (ib >> 1)) ^ C::swz_v(vrow)) * 16) + (ib & 1) * 8;
  // Group 1 keeps its O^T blocks in swapped halves: its oacc[md] holds d-block
  // md ^ MD/2.  Then both groups keep oacc[0, MD/2) and hand over
  // oacc[MD/2, MD) in the final merge with compile-time indices only (a
  // runtime index would move the accumulators to scratch memory).
  const int mdx = grp == 0 ? 0 : C::MD / 2;
  __syncthreads();  // bias table and Q tile complete
  // Q fragments, read like those of a K tile; waited for here, before the
  // first VALU slot's copies can reach the buffer.
  bf16x8 qf[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(v_s1 + w4 * 32 * C::ROW + (koff0 ^ (ks << 5)));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  {
    auto batch_count = [&](int b) __attribute__((always_inline)) {
      return ((b + 2 < niter) ? C::DMA : 0) + ((b + 1 >= 0 && b + 1 < niter) ? C::DMA : 0) + g_count(b + 3);
    };

    float m = -INFINITY;
    bool eager = false;  // this wave takes the row maxima on every tile (see the VALU slot)
    float lsum = 0.0f;
    f32x16 oacc[C::MD];
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;
    f32x16 sacc[2];
    bf16x8 pf[4];

    // K(t), V(t-1) (and g(t+1)) came with batch t-2; batch t-1 may still be landing.
    auto wait_for_tile = [&](int t) __attribute__((always_inline)) {
      const int nf = batch_count(t - 1);
      if (nf == 2 * C::DMA + 1)
        wait_vm<2 * C::DMA + 1>();
      else if (nf == 2 * C::DMA)
        wait_vm<2 * C::DMA>();
      else if (nf == C::DMA + 1)
        wait_vm<C::DMA + 1>();
      else if (nf == C::DMA)
        wait_vm<C::DMA>();
      else if (nf == 1)
        wait_vm<1>();
      else
        wait_vm<0>();
    };
    // MFMA slot t: O^T += V^T P^T for tile t-1, then S^T = bias + K Q^T for
    // tile t.  Operand fragments are double-buffered one block ahead: the
    // LDS reads for block i+1 are issued before the MFMAs of block i, so the
    // matrix core does not wait out an LDS latency per instruction.
    // sched_barrier(0) pins that order.
    auto mfma_slot = [&](int t) __attribute__((always_inline)) {
      // Higher issue priority while this wave feeds the matrix core; the
      // other wave on the SIMD (in its VALU slot) fills the gaps.
      __builtin_amdgcn_s_setprio(2);
      // STREAM: the bias of tile t+1 from its gate values (batch t-2), read
      // now and written after the PV products, so the LDS latency and the
      // log2 hide behind the matrix work.
      const bool next_bias = g_wave && t + 1 < niter;
      float g_next = 0.0f;
      if (next_bias) g_next = graw[grp][(t + 1) & 3][lane];
      if (t >= 1 && t - 1 < niter) {
        const uint8_t* vs = ((t - 1) & 1 ? v_s1 : v_s0) + grp * KB;
        bf16x8 vf[2][C::MD];
        auto load_v = [&](int kb, bf16x8* dst) __attribute__((always_inline)) {
#pragma unroll
          for (int md = 0; md < C::MD; ++md) {
            const uint8_t* vp = vs + (voff0 ^ ((md ^ mdx) << 6)) + (16 * kb) * C::ROW;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * C::ROW));
            dst[md] = __builtin_bit_cast(
                bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          }
        };
        load_v(0, vf[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb + 1 < 4) load_v(kb + 1, vf[(kb + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int md = 0; md < C::MD; ++md)
            oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb & 1][md], pf[kb], oacc[md], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (next_bias) {
        bias_s[grp][(t + 1) & 1][lane] = bias_of(t + 1, g_next);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): written before the next barrier
      }
      if (t < niter) {
        const int kt = 2 * t + grp;
        const uint8_t* ksb = (t & 1 ? k_s1 : k_s0) + grp * KB;
        // Without a gate every tile reads the 64 zeros at the start of the table
        // (keys past the prompt are then removed by the causal test).
        // A prompt longer than the host's max_seqlen (a broken precondition)
        // could reach past the table: the index is clamped into it.
        const float* bias = STREAM ? &bias_s[grp][t & 1][0] : bias_all + (has_gate ? min(kt, MAXK / BN - 1) * BN : 0);
        bf16x8 kf[2][2][2];  // [buffer][k-step within the pair][32-key half]
        auto load_k = [&](int kp, bf16x8 (*dst)[2]) __attribute__((always_inline)) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              dst[u][mb] = *reinterpret_cast<const bf16x8*>(ksb + mb * 32 * C::ROW + (koff0 ^ ((2 * kp + u) << 5)));
        };
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const f32x4 bj = *reinterpret_cast<const f32x4*>(bias + mb * 32 + 8 * rq + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[mb][4 * rq + e] = bj[e];
          }
        load_k(0, kf[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kp = 0; kp < DH / 32; ++kp) {
          if (kp + 1 < DH / 32) load_k(kp + 1, kf[(kp + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kp & 1][u][mb], qf[2 * kp + u], sacc[mb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // VALU slot t: copies for later tiles, then the online softmax of tile t.
    auto valu_slot = [&](int t) __attribute__((always_inline)) {
      if (t < 0) return;
      if (t + 2 < niter) issue(kbase, off_k, 2 * (t + 2) + grp, k_addr[t & 1]);
      if (t + 1 < niter) issue(vbase, off_v, 2 * (t + 1) + grp, v_addr[(t + 1) & 1]);
      if (t + 3 < niter) issue_g(t + 3);
      if (t >= niter) return;
      const int kt = 2 * t + grp;
      if (kt * BN + BN - 1 > row0 + w4 * 32) {  // tile reaches past this wave's first query
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = kt * BN + mb * 32 + 8 * rq + 4 * half + e;
              sacc[mb][4 * rq + e] = j > qi ? -INFINITY : sacc[mb][4 * rq + e];
            }
      }
      // p = 2^(c*s - m) against the lane's reference maximum m, packed to
      // bf16 for the PV product; returns the lane's sum of p (four partial
      // sums, so the adds do not form one serial chain).
      auto weights = [&]() __attribute__((always_inline)) {
        const float msub = (m == -INFINITY) ? 0.0f : m;
        float ps[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          ps[kb] = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb >> 1][8 * (kb & 1) + e], c, -msub));
            ps[kb] += p;
            pf[kb][e] = (__bf16)p;
          }
        }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
      };
      // The reference maximum is set from the row maxima on a wave's first
      // tile and afterwards only when a tile's weights show it too low: some
      // weight above 2^64, or a sum that overflowed or is NaN.  Until then
      // every p stays below 2^64: the fp32 sums, the bf16 weights and the O
      // accumulators keep the same relative precision as with p <= 1
      // (numerator and denominator share the shift) and stay far from the
      // fp32 range, so the row maxima are not needed.  When the check fails
      // the tile is redone against its true maxima, and from then on the wave
      // takes the row maxima on every tile (logits that outgrow the first
      // tile's maxima that far tend to keep rising, and each redo computes
      // the tile's weights twice).  A lane with no reference yet (no visible
      // key in its first tile) must see no weight either: such a lane never
      // meets a visible key later (its group's first tile covers its earliest
      // keys), and the check makes sure of it.
      constexpr float kWeightBound = 18446744073709551616.0f;  // 2^64
      float psum = 0.0f;
      bool exact = t == 0 || eager;
      if (!exact) {
        psum = weights();
        exact = __any(!(psum <= kWeightBound) || (psum > 0.0f && m == -INFINITY));
        eager = exact;
      }
      if (exact) {
        // The reference moves only when some lane's logits exceed it by more
        // than 8 (log2 units): weights stay below 2^8, and the O rescale is
        // skipped on most tiles.  A tile that failed the check always moves
        // it (some weight was above 2^64), and so does the first (m = -inf).
        float mloc = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[mb][r]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
          mloc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float m_new = fmaxf(m, mloc * c);
        if (__any(m_new > m + 8.0f)) {
          const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
          lsum *= alpha;
#pragma unroll
          for (int md = 0; md < C::MD; ++md)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
          m = m_new;
        }
        psum = weights();
      }
      lsum += psum;
    };

    // Slot pairs u = 0..niter0.  Group 0: MFMA slot u, then VALU slot u.
    // Group 1, one slot behind: VALU slot u-1, then MFMA slot u.  Both groups
    // meet the same two barriers per pair.
    if (grp == 0) {
      for (int u = 0; u <= niter0; ++u) {
        wait_for_tile(u);
        plain_barrier();
        mfma_slot(u);
        plain_barrier();
        valu_slot(u);
      }
    } else {
      for (int u = 0; u <= niter0; ++u) {
        plain_barrier();
        valu_slot(u - 1);
        wait_for_tile(u);
        plain_barrier();
        mfma_slot(u);
      }
    }

    // ---- merge the two groups' partial results, normalise, store ----
    // Group 0 finishes d-blocks md < MD/2, group 1 blocks md >= MD/2: each
    // hands the other half of its partial O^T (and its m, l) across LDS in
    // 16-byte pieces.  The normalised bf16 tile is staged in LDS (the second
    // V buffer, unused by the merge) and written out as whole rows: written
    // straight from the accumulators, every store instruction would touch 32
    // query rows.
    __syncthreads();
    constexpr int HM = C::MD / 2;
    f32x4* to_g0 = reinterpret_cast<f32x4*>(k_s0);  // group 1's rows md < HM
    f32x4* to_g1 = reinterpret_cast<f32x4*>(k_s1);  // group 0's rows md >= HM
    float* scr_m = reinterpret_cast<float*>(v_s0);
    float* scr_l = scr_m + 8 * 64;
    {
      f32x4* out = grp == 0 ? to_g1 : to_g0;
#pragma unroll
      for (int h = 0; h < HM; ++h)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          out[(w4 * (HM * 4) + h * 4 + rq) * 64 + lane] =
              f32x4{oacc[HM + h][4 * rq], oacc[HM + h][4 * rq + 1], oacc[HM + h][4 * rq + 2], oacc[HM + h][4 * rq + 3]};
      scr_m[wave * 64 + lane] = m;
      scr_l[wave * 64 + lane] = lsum;
    }
    __syncthreads();
    // Output tile in LDS: row ql = query row0 + ql, DH/8 chunks of 16 bytes,
    // chunk c stored at c ^ (ql % (DH/8)).
    uint8_t* const stage = v_s1;
    constexpr int ROWB = DH * 2;
    constexpr int CMASK = DH / 8 - 1;
    static_assert(C::BM * ROWB <= 2 * KB, "output tile fits in one V buffer pair");
    {
      const float m1 = scr_m[(wave ^ 4) * 64 + lane];
      const float l1 = scr_l[(wave ^ 4) * 64 + lane];
      const float mt_ = fmaxf(m, m1);
      const float a0 = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mt_);
      const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m1 - mt_);
      float l = lsum * a0 + l1 * a1;
      l += __shfl_xor(l, 32, kWave);
      const float inv = 1.0f / l;
      const f32x4* in = grp == 0 ? to_g0 : to_g1;
      const int md0 = grp == 0 ? 0 : HM;
      const int ql = w4 * 32 + r32;
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const f32x16& keep = oacc[h];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 iv = in[(w4 * (HM * 4) + h * 4 + rq) * 64 + lane];
          float ov[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (keep[4 * rq + e] * a0 + iv[e] * a1) * inv;
          const u32x2 packed = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
          const int c = (md0 + h) * 4 + rq;  // the 16-byte chunk holding dh 8c .. 8c+7
          *reinterpret_cast<u32x2*>(stage + ql * ROWB + ((c ^ (ql & CMASK)) << 4) + 8 * half) = packed;
        }
      }
      if (a.lse && grp == 0 && half == 0 && qi < L)
        a.lse[(int64_t)head * a.total + s0 + qi] = (mt_ + log2f(l)) * kLn2;
    }
    __syncthreads();
    {
      // 16 consecutive threads write one query row (DH = 128) with 16-byte stores.
      constexpr int CPR_O = DH / 8;
#pragma unroll
      for (int x = tid; x < C::BM * CPR_O; x += 512) {
        const int ql = x / CPR_O, c = x % CPR_O;
        if (row0 + ql < L) {
          const u32x4 val = *reinterpret_cast<const u32x4*>(stage + ql * ROWB + ((c ^ (ql & CMASK)) << 4));
          *reinterpret_cast<u32x4*>(a.o + (((s0 + row0 + ql) * hq + head) * DH) * 2 + c * 16) = val;
        }
      }
    }
  }
  };
  const int mt0 = ntiles - 1 - pair;
  if (pair >= (ntiles + 1) / 2) return;  // pairs past this prompt's tiles
  tile_body(mt0, true);
  if (pair >= mt0) return;
  __syncthreads();  // the next tile's copies reuse the LDS of this tile's merge
  tile_body(pair, false);
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per query, keys streamed through LDS in tiles of 64,
// natural-base online softmax with the ln g bias.  Causal by kept index, as the
// bf16 kernels: key j is visible to query i iff j <= i, which is the mask on
// original positions whenever they strictly increase.
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const float* __restrict__ g,
                                                      const float* __restrict__ head_gain,
                                                      float* __restrict__ o, float* __restrict__ lse,
                                                      const int32_t* __restrict__ cu, int total, int hq,
                                                      int hkv, float scale) {
  __shared__ float ks[64][DH];
  __shared__ float vs[64][DH];
  __shared__ float bs[64];
  const int lane = threadIdx.x;
  const int head = blockIdx.y;
  const int kvh = head / (hq / hkv);
  int64_t s0 = 0;
  int L = total;
  if (cu) {
    s0 = cu[blockIdx.z];
    L = cu[blockIdx.z + 1] - (int)s0;
  }
  const int q0 = blockIdx.x * 64;
  if (q0 >= L) return;
  const float gain = head_gain ? head_gain[head] : 1.0f;
  const int qi = q0 + lane;
  const int qrow = qi < L ? qi : L - 1;
  float qv[DH];
  const float* qp = q + ((s0 + qrow) * hq + head) * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) qv[d] = qp[d];
  float m = -INFINITY, l = 0.0f;
  float ov[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) ov[d] = 0.0f;
  const int kend = min(L, q0 + 64);
  for (int k0 = 0; k0 < kend; k0 += 64) {
    for (int x = lane; x < 64 * DH; x += 64) {
      const int key = x / DH, d = x % DH;
      int j = k0 + key;
      j = j < L ? j : L - 1;
      ks[key][d] = k[((s0 + j) * hkv + kvh) * DH + d];
      vs[key][d] = v[((s0 + j) * hkv + kvh) * DH + d];
    }
    {
      const int j = k0 + lane;
      bs[lane] = j < L ? (g ? logf(fmaxf(g[s0 + j], kFltMin)) * gain : 0.0f) : -INFINITY;
    }
    __syncthreads();
    const int nk = min(64, kend - k0);
    for (int jj = 0; jj < nk; ++jj) {
      if (k0 + jj > qi) break;
      float sdot = 0.0f;
#pragma unroll
      for (int d = 0; d < DH; ++d) sdot = fmaf(qv[d], ks[jj][d], sdot);
      const float sl = fmaf(sdot, scale, bs[jj]);
      const float m_new = fmaxf(m, sl);
      const float alpha = expf(m - m_new);
      const float p = expf(sl - m_new);
      l = fmaf(l, alpha, p);
#pragma unroll
      for (int d = 0; d < DH; ++d) ov[d] = fmaf(ov[d], alpha, p * vs[jj][d]);
      m = m_new;
    }
    __syncthreads();
  }
  if (qi < L) {
    const float inv = 1.0f / l;
    float* op = o + ((s0 + qi) * hq + head) * DH;
#pragma unroll
    for (int d = 0; d < DH; ++d) op[d] = ov[d] * inv;
    if (lse) lse[(int64_t)head * total + s0 + qi] = m + logf(l);
  }
}

}  // namespace

hipError_t launch_attn_bf16(int64_t total, const int32_t* cu_seqlens, int batch, int64_t max_seqlen,
                            int hq, int hkv, int dh, float scale, const void* q, const void* k,
                            const void* v, const float* g, const float* head_gain, const int32_t* pos,
                            void* o, float* lse, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.g = g;
  a.head_gain = head_gain;
  a.pos = pos;
  a.o = static_cast<uint8_t*>(o);
  a.lse = lse;
  a.cu = cu_seqlens;
  a.total = (int)total;
  a.hq = hq;
  a.hkv = hkv;
  a.scale_log2 = scale * kLog2e;
  const int64_t ntiles = (max_seqlen + 127) / 128;
  const int64_t npairs = (ntiles + 1) / 2;
  if (!grid_fits(npairs * hq, 512, cu_seqlens ? batch : 1)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(npairs * hq), cu_seqlens ? (unsigned)batch : 1u);
  // The ping-pong kernel keeps a bias entry per key (rounded up to a 64-key
  // tile) in LDS; without a gate it needs no table and takes any length.
  // Longer gated prompts take the streaming-bias kernel.  Both take the
  // same grid of tile pairs.
  const int64_t keys = (max_seqlen + 63) / 64 * 64;
  if (dh == 128) {
    if (!g || keys <= PPCfg<128>::MAXK)
      hipLaunchKernelGGL((attn_bf16_pp_kernel<128, false>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16_pp_kernel<128, true>), grid, dim3(512), 0, stream, a);
  } else {
    if (!g || keys <= PPCfg<64>::MAXK)
      hipLaunchKernelGGL((attn_bf16_pp_kernel<64, false>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16_pp_kernel<64, true>), grid, dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(int64_t total, const int32_t* cu_seqlens, int batch, int64_t max_seqlen,
                           int hq, int hkv, int dh, float scale, const float* q, const float* k,
                           const float* v, const float* g, const float* head_gain, float* o,
                           float* lse, hipStream_t stream) {
  if (!grid_fits((max_seqlen + 63) / 64, 64, hq, cu_seqlens ? batch : 1)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((max_seqlen + 63) / 64), (unsigned)hq, cu_seqlens ? (unsigned)batch : 1u);
  if (dh == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, q, k, v, g, head_gain, o,
                       lse, cu_seqlens, (int)total, hq, hkv, scale);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, g, head_gain, o,
                       lse, cu_seqlens, (int)total, hq, hkv, scale);
  return hipGetLastError();
}

}  // namespace tg
