// Decode attention over the compact KV cache on gfx950.
//
// After the gated prefill the upper layers hold keys and values only for the
// kept tokens (aitualizate.com article, section "3. Las capas superiores
// procesan únicamente los tokens seleccionados"); each generated token then
// attends once over its sequence's whole cache.  This library's reading for
// the gate bias (decode is not described on the pages): the kept prompt keys
// keep their bias gamma_h * ln max(g_j, FLT_MIN), generated tokens carry
// g = 1, and g = NULL means no bias.
//
// One new query per sequence makes the work a matrix-vector product per head:
// 16.8 MB of bf16 cache per step for 4096 keys x 8 KV heads x 128 dims, two
// flop per byte, so the kernel is bound by HBM.  Split-K over the cache:
//  * decode_split_kernel: one workgroup (4 waves) per (sequence, KV head,
//    block of S keys) handles every query head of that KV group.  A key row
//    (dh elements) is read by dh/8 consecutive lanes, 8 elements each, so the
//    reads are coalesced 16-byte loads; the q.k dot product is reduced over
//    those lanes with xor shuffles.  Every lane keeps its own online softmax
//    (reference maximum moved only when a logit exceeds it by more than 8 in
//    log2 units) and its 8 output dimensions; lanes, then waves, merge their
//    (max, sum, output) at the end, and the block's partial result goes to the
//    caller's workspace.
//  * decode_combine_kernel: one workgroup per (sequence, query head) merges
//    the partial results of the blocks and writes o and lse.
#include <cmath>

#include "tg_internal.h"

namespace tg {

int decode_split_keys(int64_t batch, int hkv, int64_t max_seqlen) {
  // Keys per block: enough blocks to fill the chip (>= ~512 workgroups) but
  // at least 64 keys each.
  int s = 1024;
  while (s > 64 && batch * hkv * ((max_seqlen + s - 1) / s) < 512) s >>= 1;
  return s;
}

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* x) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* head_gain;
  const int32_t* cu;
  float* part;  // [batch, hq, nsplit, DH + 2]: m (log2 units), l, o[DH] (not normalised)
  void* o;
  float* lse;
  int hq;
  int hkv;
  int nsplit;
  int split;
  float scale_log2;
};

// GROUP = query heads per KV head (compile-time so that per-head state stays
// in registers).
template <typename T, int DH, int GROUP>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecArgs a) {
  constexpr int LPK = DH / 8;          // lanes per key row
  constexpr int KPW = kWave / LPK;     // key rows per wave per step
  constexpr int KPB = KPW * kDecWaves; // key rows per workgroup per step
  __shared__ float red[kDecWaves][GROUP][DH + 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dc = lane % LPK;  // this lane's 8-element chunk of a row
  const int ks = lane / LPK;  // this lane's key slot within the wave
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s0 = a.cu[b];
  const int L = a.cu[b + 1] - (int)s0;
  const int k0 = split * a.split;
  if (k0 >= L) return;
  const int k1 = min(L, k0 + a.split);
  const float c = a.scale_log2;

  float qv[GROUP][8], gain[GROUP];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    const int h = kvh * GROUP + i;
    load8<T>(reinterpret_cast<const T*>(a.q) + ((int64_t)b * a.hq + h) * DH + dc * 8, qv[i]);
    gain[i] = a.head_gain ? a.head_gain[h] : 1.0f;
  }
  float m[GROUP], l[GROUP], acc[GROUP][8];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
  }

  const T* kb = reinterpret_cast<const T*>(a.k) + (s0 * a.hkv + kvh) * DH + dc * 8;
  const T* vb = reinterpret_cast<const T*>(a.v) + (s0 * a.hkv + kvh) * DH + dc * 8;
  const int64_t row = (int64_t)a.hkv * DH;  // elements between consecutive keys
  // Two steps per iteration, loads first, so that four 16-byte loads per lane
  // are in flight.
  for (int j0 = k0; j0 < k1; j0 += 2 * KPB) {
    float kx[2][8], vx[2][8];
    int jj[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      jj[u] = j0 + u * KPB + wave * KPW + ks;
      const int jr = jj[u] < k1 ? jj[u] : k1 - 1;
      load8<T>(kb + jr * row, kx[u]);
      load8<T>(vb + jr * row, vx[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float bias = a.g ? log2f(fmaxf(a.g[s0 + (jj[u] < k1 ? jj[u] : k1 - 1)], kFltMin)) : 0.0f;
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[i][e], kx[u][e], d);
#pragma unroll
        for (int o = LPK / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, kWave);
        // Logit in log2 units; rows past this block weigh nothing.
        const float t = jj[u] < k1 ? fmaf(d, c, gain[i] * bias) : -INFINITY;
        if (t > m[i] + 8.0f) {
          const float alpha = m[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[i] - t);
          l[i] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
          m[i] = t;
        }
        const float p = m[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(t - m[i]);
        l[i] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(p, vx[u][e], acc[i][e]);
      }
    }
  }

  // Merge the key slots of a wave (lanes with the same chunk dc).
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
#pragma unroll
    for (int o = LPK; o < kWave; o <<= 1) {
      const float m2 = __shfl_xor(m[i], o, kWave);
      const float l2 = __shfl_xor(l[i], o, kWave);
      const float mn = fmaxf(m[i], m2);
      const float a1 = m[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[i] - mn);
      const float a2 = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2 - mn);
      l[i] = l[i] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = acc[i][e] * a1 + __shfl_xor(acc[i][e], o, kWave) * a2;
      m[i] = mn;
    }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][i][dc * 8 + e] = acc[i][e];
      if (dc == 0) {
        red[wave][i][DH] = m[i];
        red[wave][i][DH + 1] = l[i];
      }
    }
  }
  __syncthreads();
  // Merge the waves; thread t < GROUP*DH owns (head t / DH, dimension t % DH).
  for (int t = tid; t < GROUP * (DH + 2); t += kDecThreads) {
    const int i = t / (DH + 2), d = t % (DH + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, red[w][i][DH]);
    float val = 0.0f;
    if (d == DH) {
      val = mx;
    } else {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = red[w][i][DH];
        const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mx);
        val += red[w][i][d] * f;
      }
    }
    const int h = kvh * GROUP + i;
    a.part[(((int64_t)b * a.hq + h) * a.nsplit + split) * (DH + 2) + d] = val;
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(DH) void decode_combine_kernel(DecArgs a) {
  const int d = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = a.cu[b + 1] - a.cu[b];
  const int ns = min(a.nsplit, (L + a.split - 1) / a.split);  // blocks that ran for this sequence
  const float* p = a.part + ((int64_t)b * a.hq + h) * a.nsplit * (DH + 2);
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, p[s * (DH + 2) + DH]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float ms = p[s * (DH + 2) + DH];
    const float f = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - mx);
    num = fmaf(p[s * (DH + 2) + d], f, num);
    den = fmaf(p[s * (DH + 2) + DH + 1], f, den);
  }
  const float ov = den > 0.0f ? num / den : 0.0f;  // empty cache: zeros
  const int64_t oi = ((int64_t)b * a.hq + h) * DH + d;
  if constexpr (sizeof(T) == 2) {
    __bf16 hv = (__bf16)ov;
    reinterpret_cast<__bf16*>(a.o)[oi] = hv;
  } else {
    reinterpret_cast<float*>(a.o)[oi] = ov;
  }
  if (a.lse && d == 0) a.lse[(int64_t)b * a.hq + h] = den > 0.0f ? (mx + log2f(den)) * kLn2 : -INFINITY;
}

template <typename T, int DH, int GROUP>
void launch_group(const DecArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, DH, GROUP>), dim3(a.nsplit, a.hkv, batch), dim3(kDecThreads), 0,
                     stream, a);
  hipLaunchKernelGGL((decode_combine_kernel<T, DH>), dim3(a.hq, batch), dim3(DH), 0, stream, a);
}

template <typename T, int DH>
hipError_t launch_dh(const DecArgs& a, int batch, hipStream_t stream) {
  switch (a.hq / a.hkv) {
    case 1: launch_group<T, DH, 1>(a, batch, stream); break;
    case 2: launch_group<T, DH, 2>(a, batch, stream); break;
    case 4: launch_group<T, DH, 4>(a, batch, stream); break;
    case 8: launch_group<T, DH, 8>(a, batch, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int elem_bytes, const int32_t* cu_seqlens, int batch, int64_t max_seqlen, int hq,
                         int hkv, int dh, float scale, const void* q, const void* k, const void* v,
                         const float* g, const float* head_gain, void* o, float* lse, float* workspace,
                         hipStream_t stream) {
  DecArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.head_gain = head_gain;
  a.cu = cu_seqlens;
  a.part = workspace;
  a.o = o;
  a.lse = lse;
  a.hq = hq;
  a.hkv = hkv;
  a.split = decode_split_keys(batch, hkv, max_seqlen);
  a.nsplit = (int)((max_seqlen + a.split - 1) / a.split);
  if (a.nsplit < 1) a.nsplit = 1;
  a.scale_log2 = scale * kLog2e;
  if (elem_bytes == 2)
    return dh == 128 ? launch_dh<uint16_t, 128>(a, batch, stream) : launch_dh<uint16_t, 64>(a, batch, stream);
  return dh == 128 ? launch_dh<float, 128>(a, batch, stream) : launch_dh<float, 64>(a, batch, stream);
}

}  // namespace tg
