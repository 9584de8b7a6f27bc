// Weighted combine back to token order (MoE-Prism, arXiv 2510.19366, §III-B2:
// the routed output is the router-weighted sum of the executed experts' FFNs;
// shared experts add with weight 1, §II-B):
//   out[t] = sum_{j < k_t} w[t, j] * Y[inv_perm[tok_off[t] + j]]  (+ Y_shared[t])
// in float32, j ascending (deterministic), rounded once to the element type.
// An assignment whose inv_perm entry is negative has no row and adds nothing.
#include "common.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// One workgroup per token; a thread owns 16-byte column chunks c, c+256, ...
// The rows of CB assignments are requested together, one batch ahead of the
// batch being summed; the sum runs in ascending j (the loads overlap, the
// arithmetic order does not change).
constexpr int CB = 8;

template <typename T>
__device__ __forceinline__ void load_chunk(const T* p, float (&f)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void load_chunk<bf16_t>(const bf16_t* p, float (&f)[8]) {
  unpack(*reinterpret_cast<const uint4*>(p), f);
}
template <>
__device__ __forceinline__ void load_chunk<float>(const float* p, float (&f)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
template <typename T>
__device__ __forceinline__ void unpack_chunk(const uint4& v, float (&f)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void unpack_chunk<bf16_t>(const uint4& v, float (&f)[8]) {
  unpack(v, f);
}
template <>
__device__ __forceinline__ void unpack_chunk<float>(const uint4& v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y); f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
template <typename T>
__device__ __forceinline__ void store_chunk(T* p, const float* f);
template <>
__device__ __forceinline__ void store_chunk<bf16_t>(bf16_t* p, const float* f) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(o[0], o[1], o[2], o[3]);
}
template <>
__device__ __forceinline__ void store_chunk<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const T* __restrict__ ysh,
                                                      const int32_t* __restrict__ tok_off,
                                                      const float* __restrict__ wts,
                                                      const int32_t* __restrict__ inv_perm, T* __restrict__ out,
                                                      int d) {
  constexpr int LE = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int a0 = tok_off[t], a1 = tok_off[t + 1];
  const int nb = (a1 - a0 + CB - 1) / CB;
  for (int c = threadIdx.x; c < d / LE; c += 256) {
    float acc[LE];
#pragma unroll
    for (int i = 0; i < LE; ++i) acc[i] = 0.f;
    uint4 rb[2][CB];
    auto issue = [&](uint4 (&r)[CB], int b) {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int a = a0 + b * CB + j;
        const int p = a < a1 ? inv_perm[a] : -1;  // -1: an assignment without a row
        // Y is read exactly once: non-temporal loads keep it from displacing
        // anything in the caches
        r[j] = zero_u4();
        if (p >= 0) {
          const u32x4_t v = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(y + (size_t)p * d + c * LE));
          r[j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      }
    };
    auto consume = [&](const uint4 (&r)[CB], int b) {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int a = a0 + b * CB + j;
        if (a < a1 && inv_perm[a] >= 0) {
          float f[LE];
          unpack_chunk<T>(r[j], f);
          const float w = wts[a];
#pragma unroll
          for (int i = 0; i < LE; ++i) acc[i] = fmaf(w, f[i], acc[i]);
        }
      }
    };
    if (nb > 0) issue(rb[0], 0);
    for (int b = 0; b < nb; b += 2) {
      if (b + 1 < nb) issue(rb[1], b + 1);
      consume(rb[0], b);
      if (b + 2 < nb) issue(rb[0], b + 2);
      if (b + 1 < nb) consume(rb[1], b + 1);
    }
    if (ysh) {
      float f[LE];
      load_chunk<T>(ysh + (size_t)t * d + c * LE, f);
#pragma unroll
      for (int i = 0; i < LE; ++i) acc[i] += f[i];
    }
    store_chunk<T>(out + (size_t)t * d + c * LE, acc);
  }
}

hipError_t launch_combine(int dtype, const void* y, const void* y_shared, const int32_t* tok_off,
                          const float* wts, const int32_t* inv_perm, void* out, int T, int d, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)y, (const bf16_t*)y_shared,
                       tok_off, wts, inv_perm, (bf16_t*)out, d);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)y, (const float*)y_shared,
                       tok_off, wts, inv_perm, (float*)out, d);
  return hipGetLastError();
}

}  // namespace moe
