// Stage 5 -- RoPE at the kept tokens' original positions and the compact KV
// cache, on gfx950.
//
// aitualizate.com article, section "3. Las capas superiores procesan
// únicamente los tokens seleccionados": discarded tokens create no key/value
// cache entries in the layers above L, so the cache holds exactly the K kept
// tokens.  Position encoding is not described on the pages; this library
// uses rotate-half RoPE (pairs (i, i + dh/2), angle pos * base^(-2i/dh)) at
// each kept token's position in the original prompt.
//
// The cos/sin table is built once per (max_pos, dh, base) in fp64 on the
// device and stored as fp32; the rotation itself runs in fp32 and rounds once
// to the storage type.  One workgroup per kept token: it rotates the token's
// query heads in place, writes its rotated keys to k_cache and copies its
// values to v_cache, 16-byte accesses throughout.
#include "tg_internal.h"

namespace tg {
namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ cs, int64_t max_pos,
                                                         int dh, double base) {
  const int half = dh / 2;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= max_pos * half) return;
  const int64_t p = t / half;
  const int i = (int)(t - p * half);
  const double theta = pow(base, -2.0 * (double)i / (double)dh);
  const double phi = (double)p * theta;
  cs[p * dh + i] = (float)cos(phi);
  cs[p * dh + half + i] = (float)sin(phi);
}

// Storage helpers: 8 consecutive elements <-> 8 floats.
template <int ES>
struct Vec8;
template <>
struct Vec8<2> {  // bf16
  static __device__ __forceinline__ void load(const void* p, float* f) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* p, const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = v;
  }
};
template <>
struct Vec8<4> {  // fp32
  static __device__ __forceinline__ void load(const void* p, float* f) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(void* p, const float* f) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = f[i];
      b[i] = f[4 + i];
    }
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
  }
};

template <int ES>
__global__ __launch_bounds__(256) void rope_kv_kernel(int hq, int hkv, int dh,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ cs, int64_t max_pos,
                                                      uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ k,
                                                      const uint8_t* __restrict__ v,
                                                      uint8_t* __restrict__ kc,
                                                      uint8_t* __restrict__ vc) {
  const int64_t tok = blockIdx.x;
  const int p = pos[tok];
  const bool ok = p >= 0 && p < max_pos;
  const int half = dh / 2;
  const int pchunks = half / 8;                 // 8-pair chunks per head
  const int q_units = hq * pchunks;
  const int k_units = hkv * pchunks;
  const int v_units = (int)((int64_t)hkv * dh * ES / 16);
  const int64_t row_bytes = (int64_t)dh * ES;
  const float* crow = cs + (int64_t)(ok ? p : 0) * dh;
  const bool copy_v = (vc != v);

  for (int u = threadIdx.x; u < q_units + k_units + (copy_v ? v_units : 0); u += blockDim.x) {
    if (u < q_units + k_units) {
      const bool is_q = u < q_units;
      const int uu = is_q ? u : u - q_units;
      const int head = uu / pchunks;
      const int c = uu - head * pchunks;
      const int64_t rb = (tok * (is_q ? hq : hkv) + head) * row_bytes;
      const uint8_t* src = (is_q ? q : k) + rb;
      uint8_t* dst = (is_q ? q : kc) + rb;
      float x1[8], x2[8], y1[8], y2[8];
      Vec8<ES>::load(src + (int64_t)c * 8 * ES, x1);
      Vec8<ES>::load(src + (int64_t)(half + c * 8) * ES, x2);
      if (ok) {
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(crow + c * 8);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(crow + c * 8 + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(crow + half + c * 8);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(crow + half + c * 8 + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float co = i < 4 ? c0[i] : c1[i - 4];
          const float si = i < 4 ? s0[i] : s1[i - 4];
          y1[i] = x1[i] * co - x2[i] * si;
          y2[i] = x2[i] * co + x1[i] * si;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y1[i] = y2[i] = 0.0f;
      }
      Vec8<ES>::store(dst + (int64_t)c * 8 * ES, y1);
      Vec8<ES>::store(dst + (int64_t)(half + c * 8) * ES, y2);
    } else {
      const int c = u - q_units - k_units;
      const int64_t o = tok * hkv * row_bytes + (int64_t)c * 16;
      const u32x4 val = ok ? *reinterpret_cast<const u32x4*>(v + o) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(vc + o) = val;
    }
  }
}

}  // namespace

hipError_t launch_rope_table(float* cos_sin, int64_t max_pos, int dh, double base,
                             hipStream_t stream) {
  const int64_t total = max_pos * (dh / 2);
  if (!grid_fits((total + 255) / 256, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     cos_sin, max_pos, dh, base);
  return hipGetLastError();
}

hipError_t launch_rope_kv(int elem_bytes, int64_t n_kept, int hq, int hkv, int dh, const int32_t* pos,
                          const float* cos_sin, int64_t max_pos, void* q, const void* k, const void* v,
                          void* k_cache, void* v_cache, hipStream_t stream) {
  if (!grid_fits(n_kept, 256)) return hipErrorInvalidConfiguration;
  auto* qb = static_cast<uint8_t*>(q);
  auto* kb = static_cast<const uint8_t*>(k);
  auto* vb = static_cast<const uint8_t*>(v);
  auto* kcb = static_cast<uint8_t*>(k_cache);
  auto* vcb = static_cast<uint8_t*>(v_cache);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(rope_kv_kernel<2>, dim3((unsigned)n_kept), dim3(256), 0, stream, hq, hkv, dh, pos,
                       cos_sin, max_pos, qb, kb, vb, kcb, vcb);
  else
    hipLaunchKernelGGL(rope_kv_kernel<4>, dim3((unsigned)n_kept), dim3(256), 0, stream, hq, hkv, dh, pos,
                       cos_sin, max_pos, qb, kb, vb, kcb, vcb);
  return hipGetLastError();
}

}  // namespace tg
