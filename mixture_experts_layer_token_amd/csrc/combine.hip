// Weighted combine back to token order:
//   out[t] = sum_{j < k_t} w[t, j] * Y[inv_perm[tok_off[t] + j]]  (+ Y_shared[t])
// in float32, j ascending (deterministic), rounded once to the element type.
// One workgroup per token; each thread owns 16-byte column chunks.
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

__global__ __launch_bounds__(256) void combine_bf16_kernel(const bf16_t* __restrict__ y,
                                                           const bf16_t* __restrict__ ysh,
                                                           const int32_t* __restrict__ tok_off,
                                                           const float* __restrict__ wts,
                                                           const int32_t* __restrict__ inv_perm,
                                                           bf16_t* __restrict__ out, int d) {
  const int t = blockIdx.x;
  const int a0 = tok_off[t], a1 = tok_off[t + 1];
  for (int c = threadIdx.x; c < d / 8; c += 256) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int a = a0; a < a1; ++a) {
      const float w = wts[a];
      const uint4 v = *reinterpret_cast<const uint4*>(y + (size_t)inv_perm[a] * d + c * 8);
      float f[8];
      unpack(v, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, f[i], acc[i]);
    }
    if (ysh) {
      const uint4 v = *reinterpret_cast<const uint4*>(ysh + (size_t)t * d + c * 8);
      float f[8];
      unpack(v, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * d + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y, const float* __restrict__ ysh,
                                                          const int32_t* __restrict__ tok_off,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ inv_perm,
                                                          float* __restrict__ out, int d) {
  const int t = blockIdx.x;
  const int a0 = tok_off[t], a1 = tok_off[t + 1];
  for (int c = threadIdx.x; c < d / 4; c += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int a = a0; a < a1; ++a) {
      const float w = wts[a];
      const float4 v = *reinterpret_cast<const float4*>(y + (size_t)inv_perm[a] * d + c * 4);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    if (ysh) {
      const float4 v = *reinterpret_cast<const float4*>(ysh + (size_t)t * d + c * 4);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + (size_t)t * d + c * 4) = acc;
  }
}

hipError_t launch_combine(int dtype, const void* y, const void* y_shared, const int32_t* tok_off,
                          const float* wts, const int32_t* inv_perm, void* out, int T, int d, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(T), dim3(256), 0, st, (const bf16_t*)y, (const bf16_t*)y_shared,
                       tok_off, wts, inv_perm, (bf16_t*)out, d);
  else
    hipLaunchKernelGGL(combine_f32_kernel, dim3(T), dim3(256), 0, st, (const float*)y, (const float*)y_shared,
                       tok_off, wts, inv_perm, (float*)out, d);
  return hipGetLastError();
}

}  // namespace moe
