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

#include <mutex>

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

// Raw 8-element chunk of a row: one 16-byte load for bf16, two for fp32.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void to_f32(float* x) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void to_f32(float* x) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
};

// DPP lane moves within a row of 16 lanes (quad permutations and mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over each aligned group of N lanes (N = 8 or 16), result in every lane.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of each 8 lanes
  if constexpr (N == 16) x += dpp<0x140>(x);  // row_mirror: the other half of the row
  return x;
}

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* head_gain;
  const int32_t* cu;
  float* part_o;   // [batch, hq, nsplit, DH]: block outputs, not normalised
  float* part_ml;  // [batch, hq, nsplit, 2]: block maximum (log2 units) and sum
  void* o;
  float* lse;
  int hq;
  int hkv;
  int nsplit;
  int split;
  float scale_log2;
};

// GROUP = query heads per KV head (compile-time so that per-head state stays
// in registers).  U = steps (of KPB keys) per loop iteration; the loads of
// the next iteration are in flight while the current one is computed.
// NW waves per workgroup.  FINAL: the workgroup holds the sequence's whole
// cache (one block per sequence and KV head) and writes o and lse itself.
template <typename T, int DH, int GROUP, int U, int NW, bool FINAL>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecArgs a) {
  constexpr int LPK = DH / 8;          // lanes per key row
  constexpr int KPW = kWave / LPK;     // key rows per wave per step
  constexpr int KPB = KPW * NW;        // key rows per workgroup per step
  constexpr int NT = NW * 64;
  __shared__ float red[NW][GROUP][DH + 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dc = lane % LPK;  // this lane's 8-element chunk of a row
  const int ks = lane / LPK;  // this lane's key slot within the wave
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s0 = a.cu[b];
  const int L = a.cu[b + 1] - (int)s0;
  const int k0 = split * a.split;
  if (k0 >= L) {
    if (FINAL) {  // empty cache: o = 0, lse = -inf
      for (int t = tid; t < GROUP * DH; t += NT) {
        const int64_t oi = ((int64_t)b * a.hq + kvh * GROUP + t / DH) * DH + t % DH;
        if constexpr (sizeof(T) == 2)
          reinterpret_cast<__bf16*>(a.o)[oi] = (__bf16)0.0f;
        else
          reinterpret_cast<float*>(a.o)[oi] = 0.0f;
      }
      if (a.lse && tid < GROUP) a.lse[(int64_t)b * a.hq + kvh * GROUP + tid] = -INFINITY;
    }
    return;
  }
  const int k1 = min(L, k0 + a.split);
  const float c = a.scale_log2;

  const T* kb = reinterpret_cast<const T*>(a.k) + (s0 * a.hkv + kvh) * DH + dc * 8;
  const T* vb = reinterpret_cast<const T*>(a.v) + (s0 * a.hkv + kvh) * DH + dc * 8;
  // Gate values; with no gate the loads read a valid dummy word (cu) and the
  // value is replaced by 1, so that no load sits in a branch.
  const bool has_g = a.g != nullptr;
  const float* gb = has_g ? a.g + s0 : reinterpret_cast<const float*>(a.cu);
  const int64_t row = (int64_t)a.hkv * DH;  // elements between consecutive keys
  const int my = wave * KPW + ks;           // this lane's key within a step

  Raw8<T> rk[U], rv[U];
  float rg[U];
  auto issue = [&](int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jr = min(j0 + u * KPB + my, k1 - 1);  // past the block: reload its last row
      rk[u].load(kb + jr * row);
      rv[u].load(vb + jr * row);
      const float gl = gb[has_g ? jr : 0];
      rg[u] = has_g ? gl : 1.0f;
    }
  };
  issue(k0);

  float qv[GROUP][8], gain[GROUP];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    const int h = kvh * GROUP + i;
    Raw8<T> rq;
    rq.load(reinterpret_cast<const T*>(a.q) + ((int64_t)b * a.hq + h) * DH + dc * 8);
    rq.to_f32(qv[i]);
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

  for (int j0 = k0; j0 < k1; j0 += U * KPB) {
    float kx[U][8], vx[U][8], bias[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      rk[u].to_f32(kx[u]);
      rv[u].to_f32(vx[u]);
      bias[u] = log2f(fmaxf(rg[u], kFltMin));  // g = 1 (no gate) gives 0
    }
    if (j0 + U * KPB < k1) issue(j0 + U * KPB);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = j0 + u * KPB + my < k1;
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[i][e], kx[u][e], d);
        d = group_sum<LPK>(d);
        // Logit in log2 units; rows past this block weigh nothing.
        const float t = live ? fmaf(d, c, gain[i] * bias[u]) : -INFINITY;
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
  // Merge the waves: thread t handles (head t / (DH + 2), entry t % (DH + 2)),
  // entries DH and DH + 1 being the maximum and the sum.
  for (int t = tid; t < GROUP * (DH + 2); t += NT) {
    const int i = t / (DH + 2), d = t % (DH + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[w][i][DH]);
    float val = mx, lt = 0.0f;
    if (d != DH) {
      val = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = red[w][i][DH];
        const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mx);
        val += red[w][i][d] * f;
        if (FINAL) lt += red[w][i][DH + 1] * f;
      }
    } else if (FINAL) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = red[w][i][DH];
        lt += mw == -INFINITY ? 0.0f : red[w][i][DH + 1] * __builtin_amdgcn_exp2f(mw - mx);
      }
    }
    const int h = kvh * GROUP + i;
    if (FINAL) {
      if (d < DH) {
        const float ov = lt > 0.0f ? val / lt : 0.0f;
        const int64_t oi = ((int64_t)b * a.hq + h) * DH + d;
        if constexpr (sizeof(T) == 2)
          reinterpret_cast<__bf16*>(a.o)[oi] = (__bf16)ov;
        else
          reinterpret_cast<float*>(a.o)[oi] = ov;
      } else if (d == DH && a.lse) {
        a.lse[(int64_t)b * a.hq + h] = lt > 0.0f ? (mx + log2f(lt)) * kLn2 : -INFINITY;
      }
    } else {
      const int64_t slot = ((int64_t)b * a.hq + h) * a.nsplit + split;
      if (d < DH)
        a.part_o[slot * DH + d] = val;
      else
        a.part_ml[slot * 2 + (d - DH)] = val;
    }
  }
}

template <int N>
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* scratch) {
  // N threads (64 or 128); scratch holds N / 64 floats.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o, kWave);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if constexpr (N == 64) {
    return x;
  } else {
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
    __syncthreads();
    return is_max ? fmaxf(scratch[0], scratch[1]) : scratch[0] + scratch[1];
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(DH) void decode_combine_kernel(DecArgs a) {
  constexpr int CH = 512;  // block weights staged in LDS per chunk
  __shared__ float wts[CH];
  __shared__ float scr[2];
  const int d = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = a.cu[b + 1] - a.cu[b];
  const int ns = min(a.nsplit, (L + a.split - 1) / a.split);  // blocks that ran for this sequence
  const int64_t base = ((int64_t)b * a.hq + h) * a.nsplit;
  const float* po = a.part_o + base * DH;
  const float* pml = a.part_ml + base * 2;
  float mx = -INFINITY;
  for (int s = d; s < ns; s += DH) mx = fmaxf(mx, pml[2 * s]);
  mx = block_reduce<DH>(mx, true, scr);
  float num = 0.0f, den = 0.0f;
  for (int c0 = 0; c0 < ns; c0 += CH) {
    const int n = min(CH, ns - c0);
    __syncthreads();
    for (int s = d; s < n; s += DH) {
      const float ms = pml[2 * (c0 + s)];
      const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - mx);
      wts[s] = w;
      den = fmaf(w, pml[2 * (c0 + s) + 1], den);
    }
    __syncthreads();
    const float* pc = po + (int64_t)c0 * DH + d;
    int s = 0;
    for (; s + 8 <= n; s += 8) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = pc[(s + e) * DH];
#pragma unroll
      for (int e = 0; e < 8; ++e) num = fmaf(wts[s + e], x[e], num);
    }
    for (; s < n; ++s) num = fmaf(wts[s], pc[s * DH], num);
  }
  den = block_reduce<DH>(den, false, scr);
  const float ov = den > 0.0f ? num / den : 0.0f;  // empty cache: zeros
  const int64_t oi = ((int64_t)b * a.hq + h) * DH + d;
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<__bf16*>(a.o)[oi] = (__bf16)ov;
  } else {
    reinterpret_cast<float*>(a.o)[oi] = ov;
  }
  if (a.lse && d == 0) a.lse[(int64_t)b * a.hq + h] = den > 0.0f ? (mx + log2f(den)) * kLn2 : -INFINITY;
}

template <typename T, int DH, int GROUP>
void launch_group(DecArgs a, int batch, int64_t max_seqlen, hipStream_t stream) {
  if constexpr (GROUP <= 2) {  // 16 waves of this kernel fit the registers only for 1-2 heads per KV head
    if ((int64_t)batch * a.hkv >= 256) {
      // Enough (sequence, KV head) pairs to fill the chip with one 16-wave
      // workgroup each: no key split, no combine pass.
      a.split = (int)(max_seqlen > 0 ? max_seqlen : 1);
      a.nsplit = 1;
      hipLaunchKernelGGL((decode_split_kernel<T, DH, GROUP, 2, 16, true>), dim3(1, a.hkv, batch), dim3(1024), 0,
                         stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((decode_split_kernel<T, DH, GROUP, 2, kDecWaves, false>), dim3(a.nsplit, a.hkv, batch),
                     dim3(kDecThreads), 0, stream, a);
  hipLaunchKernelGGL((decode_combine_kernel<T, DH>), dim3(a.hq, batch), dim3(DH), 0, stream, a);
}

template <typename T, int DH>
hipError_t launch_dh(const DecArgs& a, int batch, int64_t max_seqlen, hipStream_t stream) {
  switch (a.hq / a.hkv) {
    case 1: launch_group<T, DH, 1>(a, batch, max_seqlen, stream); break;
    case 2: launch_group<T, DH, 2>(a, batch, max_seqlen, stream); break;
    case 4: launch_group<T, DH, 4>(a, batch, max_seqlen, stream); break;
    case 8: launch_group<T, DH, 8>(a, batch, max_seqlen, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// ---- workspace for the entry point that allocates nothing ----------------
// A file-scope device array (each device holds its own copy, at its own
// address, until the process ends).  Host code never passes `scratch`
// itself to a kernel: on the host that name is a stand-in, not a device
// address.  The address of each device's copy is looked up once, with that
// device current, and kept.
static __device__ __align__(256) uint8_t scratch[kDecodeStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

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
  a.part_o = workspace;
  a.o = o;
  a.lse = lse;
  a.hq = hq;
  a.hkv = hkv;
  a.split = decode_split_keys(batch, hkv, max_seqlen);
  a.nsplit = (int)((max_seqlen + a.split - 1) / a.split);
  if (a.nsplit < 1) a.nsplit = 1;
  // Split blocks over (split, KV head, sequence), combine blocks over (query head, sequence).
  if (!grid_fits(a.nsplit, kDecThreads, hkv, batch) || !grid_fits(hq, dh, batch))
    return hipErrorInvalidConfiguration;
  a.part_ml = workspace + (int64_t)batch * hq * a.nsplit * dh;
  a.scale_log2 = scale * kLog2e;
  if (elem_bytes == 2)
    return dh == 128 ? launch_dh<uint16_t, 128>(a, batch, max_seqlen, stream)
                     : launch_dh<uint16_t, 64>(a, batch, max_seqlen, stream);
  return dh == 128 ? launch_dh<float, 128>(a, batch, max_seqlen, stream)
                   : launch_dh<float, 64>(a, batch, max_seqlen, stream);
}

}  // namespace tg
