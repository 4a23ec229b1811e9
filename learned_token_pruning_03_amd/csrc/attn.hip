// Stage 4 -- token-gated causal GQA attention over the kept tokens, gfx950.
//
// TokenGate paper page (thelatestinai.com), Figure 1(c): every attention
// weight is multiplied by the gate value g_j of its key (and the weights
// renormalised); the page's Abstract and the aitualizate.com article, section
// "Cómo consigue entrenar una selección top-K": the importance score is a
// bias on the attention logits.  Both give softmax_j(scale*q.k_j + ln g_j).
// In base 2:  t_ij = (scale*log2 e) * q_i.k_j + log2 max(g_j, FLT_MIN),
// p_ij = 2^(t_ij - m_i), which is one FMA per logit; the bias enters the
// running maximum and the running sum like any other part of the logit.
//
// bf16 kernel layout (one workgroup = 512 threads = 8 waves):
//  * a workgroup owns one query head and a pair of 128-query tiles, tile
//    (T-1-p) then tile p, so that every workgroup has the same causal work;
//  * the two 4-wave groups split each tile's key range (group 0 takes the
//    even 64-key tiles, group 1 the odd ones) and merge their partial
//    (max, sum, output) through LDS at the end of the tile;
//  * inside a group each wave owns 32 queries.  S^T = K Q^T runs on
//    v_mfma_f32_32x32x16_bf16 with Q held in registers as the B operand, so
//    each lane ends up owning one query: the row max, row sum and rescale
//    are per-lane scalars, and P^T leaves the accumulators directly as the B
//    operand of O^T = V^T P^T (no LDS round trip for P);
//  * K is staged row-major and V transposed in LDS (padded rows, no bank
//    conflicts for the fragment reads), double-buffered, the next tile
//    prefetched into registers during the current tile's MFMAs;
//  * blockIdx -> (KV head, query head) is arranged so that all query heads
//    of one KV head land on the same XCD and share its L2.
#include <cmath>

#include "tg_internal.h"

namespace tg {
namespace {

struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* g;
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
  static constexpr int KROW = DH * 2 + 16;       // padded LDS bytes per K row
  static constexpr int VROW = BN * 2 + 8;        // padded LDS bytes per V^T row
  static constexpr int K_BYTES = BN * KROW;
  static constexpr int V_BYTES = DH * VROW;
  static constexpr int STAGE = K_BYTES + V_BYTES + BN * 8;  // + bias f32 + pos i32
  static constexpr int GROUP_BYTES = 2 * STAGE;
  static constexpr int LDS_BYTES = 2 * GROUP_BYTES;
  static constexpr int KL = BN * CPR / 256;      // K chunks per group thread
  static constexpr int VP = CPR / 8;             // V chunk columns per thread (x2 keys)
  static constexpr int MD = DH / 32;             // 32-row blocks of O^T
  static_assert(4 * 64 * (DH / 2 + 2) * 4 <= LDS_BYTES, "merge scratch must fit");
};

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int DH>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  using C = AttnCfg<DH>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;
  const int w4 = wave & 3;
  const int gtid = tid & 255;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int hq = a.hq, hkv = a.hkv, group = hq / hkv;
  const int rr = blockIdx.x % hq;
  const int pair = blockIdx.x / hq;
  const int kvh = rr % hkv;
  const int head = kvh * group + rr / hkv;
  int64_t s0 = 0;
  int L = a.total;
  if (a.cu) {
    s0 = a.cu[blockIdx.y];
    L = a.cu[blockIdx.y + 1] - (int)s0;
  }
  const int ntiles = (L + C::BM - 1) / C::BM;
  if (pair >= (ntiles + 1) / 2) return;

  const uint8_t* kbase = a.k + ((s0 * hkv + kvh) * DH) * 2;
  const uint8_t* vbase = a.v + ((s0 * hkv + kvh) * DH) * 2;
  const int64_t kv_stride = (int64_t)hkv * DH * 2;  // bytes between consecutive keys
  uint8_t* gbase = lds + grp * C::GROUP_BYTES;

  // Prefetch registers for one K/V tile (per group thread).
  u32x4 kreg[C::KL];
  u32x4 vreg[2 * C::VP];
  float breg = 0.0f;
  int preg = 0;

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int key = gtid / C::CPR + i * (256 / C::CPR);
      const int c = gtid % C::CPR;
      int j = kt * C::BN + key;
      j = j < L ? j : L - 1;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + j * kv_stride + c * 16);
    }
#pragma unroll
    for (int i = 0; i < C::VP; ++i) {
      const int kp = gtid & 31;
      const int c = (gtid >> 5) + 8 * i;
      int j0 = kt * C::BN + 2 * kp;
      int j1 = j0 + 1;
      j0 = j0 < L ? j0 : L - 1;
      j1 = j1 < L ? j1 : L - 1;
      vreg[2 * i] = *reinterpret_cast<const u32x4*>(vbase + j0 * kv_stride + c * 16);
      vreg[2 * i + 1] = *reinterpret_cast<const u32x4*>(vbase + j1 * kv_stride + c * 16);
    }
    if (gtid < C::BN) {
      const int j = kt * C::BN + gtid;
      if (j < L) {
        breg = log2f(fmaxf(a.g[s0 + j], kFltMin));
        preg = a.pos[s0 + j];
      } else {
        breg = -INFINITY;
        preg = 0x7fffffff;
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* sb = gbase + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int key = gtid / C::CPR + i * (256 / C::CPR);
      const int c = gtid % C::CPR;
      *reinterpret_cast<u32x4*>(sb + key * C::KROW + c * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VP; ++i) {
      const int kp = gtid & 31;
      const int c = (gtid >> 5) + 8 * i;
      uint8_t* vt = sb + C::K_BYTES + (8 * c) * C::VROW + kp * 4;
      const u32x4 x0 = vreg[2 * i], x1 = vreg[2 * i + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t*>(vt + (2 * e) * C::VROW) = lo16x2(x0[e], x1[e]);
        *reinterpret_cast<uint32_t*>(vt + (2 * e + 1) * C::VROW) = hi16x2(x0[e], x1[e]);
      }
    }
    if (gtid < C::BN) {
      reinterpret_cast<float*>(sb + C::K_BYTES + C::V_BYTES)[gtid] = breg;
      reinterpret_cast<int*>(sb + C::K_BYTES + C::V_BYTES + C::BN * 4)[gtid] = preg;
    }
  };

  for (int which = 0; which < 2; ++which) {
    const int mt = which == 0 ? ntiles - 1 - pair : pair;
    if (which == 1 && mt == ntiles - 1 - pair) break;  // middle tile of an odd count

    const int row0 = mt * C::BM;
    const int qi = row0 + w4 * 32 + r32;
    const int qrow = qi < L ? qi : L - 1;
    const uint8_t* qp = a.q + (((s0 + qrow) * hq + head) * DH) * 2;
    bf16x8 qf[DH / 16];
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + (ks * 16 + half * 8) * 2);
    const int pos_i = a.pos[s0 + qrow];

    const int kend = min(L, row0 + C::BM);
    const int n_kt = (kend + C::BN - 1) / C::BN;
    const int niter = (n_kt + 1) / 2;

    float m = -INFINITY;
    float lsum = 0.0f;
    f32x16 oacc[C::MD];
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] = 0.0f;

    if (grp < n_kt) {
      load_tile(grp);
      store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < niter; ++it) {
      const int kt = 2 * it + grp;
      const int nxt = kt + 2;
      if (nxt < n_kt) load_tile(nxt);
      if (kt < n_kt) {
        const uint8_t* sb = gbase + (it & 1) * C::STAGE;
        // ---- S^T = K Q^T for 64 keys x this wave's 32 queries ----
        f32x16 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < DH / 16; ++ks) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sb + (mb * 32 + r32) * C::KROW +
                                                               (ks * 16 + half * 8) * 2);
            sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mb], 0, 0, 0);
          }
        }
        // ---- gated logits, online softmax (base 2) ----
        const float* bias = reinterpret_cast<const float*>(sb + C::K_BYTES + C::V_BYTES);
        const int* kpos = reinterpret_cast<const int*>(sb + C::K_BYTES + C::V_BYTES + C::BN * 4);
        const bool masked_tile = kt * C::BN + C::BN - 1 > row0 + w4 * 32;
        float mloc = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int j0 = mb * 32 + 8 * rq + 4 * half;  // 4 consecutive keys
            const f32x4 bj = *reinterpret_cast<const f32x4*>(bias + j0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = fmaf(sacc[mb][4 * rq + e], a.scale_log2, bj[e]);
              if (masked_tile && kpos[j0 + e] > pos_i) x = -INFINITY;
              sacc[mb][4 * rq + e] = x;
              mloc = fmaxf(mloc, x);
            }
          }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float m_new = fmaxf(m, mloc);
        const float msub = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - msub);
        float psum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(sacc[mb][r] - msub);
            sacc[mb][r] = p;
            psum += p;
          }
        lsum = fmaf(lsum, alpha, psum);
        m = m_new;
#pragma unroll
        for (int md = 0; md < C::MD; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          bf16x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sacc[kb >> 1][8 * (kb & 1) + e];
#pragma unroll
          for (int md = 0; md < C::MD; ++md) {
            const uint8_t* vrow = sb + C::K_BYTES + (md * 32 + r32) * C::VROW;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (kb * 16 + 4 * half) * 2);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (kb * 16 + 8 + 4 * half) * 2);
            const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
            oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf,
                                                              oacc[md], 0, 0, 0);
          }
        }
      }
      if (nxt < n_kt) store_tile((it + 1) & 1);
      __syncthreads();
    }

    // ---- merge the two groups' partial results, normalise, store ----
    float* scr = reinterpret_cast<float*>(lds);
    float* scr_m = scr + 4 * 64 * (DH / 2);
    float* scr_l = scr_m + 4 * 64;
    if (grp == 1) {
#pragma unroll
      for (int md = 0; md < C::MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) scr[(w4 * (DH / 2) + md * 16 + r) * 64 + lane] = oacc[md][r];
      scr_m[w4 * 64 + lane] = m;
      scr_l[w4 * 64 + lane] = lsum;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = scr_m[w4 * 64 + lane];
      const float l1 = scr_l[w4 * 64 + lane];
      const float mt_ = fmaxf(m, m1);
      const float a0 = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mt_);
      const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m1 - mt_);
      float l = lsum * a0 + l1 * a1;
      l += __shfl_xor(l, 32, kWave);
      const float inv = 1.0f / l;
      if (qi < L) {
        uint8_t* op = a.o + (((s0 + qi) * hq + head) * DH) * 2;
#pragma unroll
        for (int md = 0; md < C::MD; ++md)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float ov[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * rq + e;
              ov[e] = (oacc[md][r] * a0 + scr[(w4 * (DH / 2) + md * 16 + r) * 64 + lane] * a1) * inv;
            }
            const u32x2 packed = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
            *reinterpret_cast<u32x2*>(op + (md * 32 + 8 * rq + 4 * half) * 2) = packed;
          }
        if (a.lse && half == 0) a.lse[(int64_t)head * a.total + s0 + qi] = (mt_ + log2f(l)) * kLn2;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per query, keys streamed through LDS in tiles of 64,
// natural-base online softmax with the ln g bias.
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const float* __restrict__ g,
                                                      const int32_t* __restrict__ pos,
                                                      float* __restrict__ o, float* __restrict__ lse,
                                                      const int32_t* __restrict__ cu, int total, int hq,
                                                      int hkv, float scale) {
  __shared__ float ks[64][DH];
  __shared__ float vs[64][DH];
  __shared__ float bs[64];
  __shared__ int ps[64];
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
  const int qi = q0 + lane;
  const int qrow = qi < L ? qi : L - 1;
  float qv[DH];
  const float* qp = q + ((s0 + qrow) * hq + head) * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) qv[d] = qp[d];
  const int pos_i = pos[s0 + qrow];
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
      bs[lane] = j < L ? logf(fmaxf(g[s0 + j], kFltMin)) : -INFINITY;
      ps[lane] = j < L ? pos[s0 + j] : 0x7fffffff;
    }
    __syncthreads();
    const int nk = min(64, kend - k0);
    for (int jj = 0; jj < nk; ++jj) {
      if (ps[jj] > pos_i) continue;
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
                            const void* v, const float* g, const int32_t* pos, void* o, float* lse,
                            hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.g = g;
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
  const dim3 grid((unsigned)(npairs * hq), cu_seqlens ? (unsigned)batch : 1u);
  if (dh == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(int64_t total, const int32_t* cu_seqlens, int batch, int64_t max_seqlen,
                           int hq, int hkv, int dh, float scale, const float* q, const float* k,
                           const float* v, const float* g, const int32_t* pos, float* o, float* lse,
                           hipStream_t stream) {
  const dim3 grid((unsigned)((max_seqlen + 63) / 64), (unsigned)hq, cu_seqlens ? (unsigned)batch : 1u);
  if (dh == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, q, k, v, g, pos, o, lse,
                       cu_seqlens, (int)total, hq, hkv, scale);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, g, pos, o, lse,
                       cu_seqlens, (int)total, hq, hkv, scale);
  return hipGetLastError();
}

}  // namespace tg
