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
// The rows of CBN assignments (CB, or 16 where budgets are larger) are
// requested together; the sum runs in ascending j (the loads overlap, the
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
__device__ __forceinline__ void store_chunk_nt(T* p, const float* f);
template <>
__device__ __forceinline__ void store_chunk_nt<bf16_t>(bf16_t* p, const float* f) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(p));
}
template <>
__device__ __forceinline__ void store_chunk_nt<float>(float* p, const float* f) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(f[i]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(p));
}

// A thread takes CC column chunks at a time (c, c + 256, ..., c + 256 (CC -
// 1)): the rows of a batch are requested for all of them before any is summed,
// so a token whose k_t fits one batch waits for memory once per CC chunks,
// not once per chunk.  The launch picks CC from d (1 where a thread has one
// chunk: more would only cost registers).  The output rows are stored with
// the non-temporal hint (nothing reads them back in the layer).
template <typename T, int CC, int CBN = CB>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const T* __restrict__ ysh,
                                                      const int32_t* __restrict__ tok_off,
                                                      const float* __restrict__ wts,
                                                      const int32_t* __restrict__ inv_perm, T* __restrict__ out,
                                                      int d) {
  constexpr int LE = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int a0 = tok_off[t], a1 = tok_off[t + 1];
  const int nch = d / LE;
  for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * CC) {
    float acc[CC][LE];
#pragma unroll
    for (int q = 0; q < CC; ++q)
#pragma unroll
      for (int i = 0; i < LE; ++i) acc[q][i] = 0.f;
    for (int b = a0; b < a1; b += CBN) {
      uint4 r[CBN][CC];
#pragma unroll
      for (int j = 0; j < CBN; ++j) {
        const int a = b + j;
        const int p = a < a1 ? inv_perm[a] : -1;  // -1: an assignment without a row
#pragma unroll
        for (int q = 0; q < CC; ++q) {
          const int c = c0 + 256 * q;
          r[j][q] = zero_u4();
          // Y is read exactly once: non-temporal loads keep it from displacing
          // anything in the caches
          if (p >= 0 && c < nch) {
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(y + (size_t)p * d + c * LE));
            r[j][q] = make_uint4(v[0], v[1], v[2], v[3]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CBN; ++j) {
        const int a = b + j;
        if (a < a1 && inv_perm[a] >= 0) {
          const float w = wts[a];
#pragma unroll
          for (int q = 0; q < CC; ++q) {
            float f[LE];
            unpack_chunk<T>(r[j][q], f);
#pragma unroll
            for (int i = 0; i < LE; ++i) acc[q][i] = fmaf(w, f[i], acc[q][i]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < CC; ++q) {
      const int c = c0 + 256 * q;
      if (c < nch) {
        if (ysh) {
          float f[LE];
          load_chunk<T>(ysh + (size_t)t * d + c * LE, f);
#pragma unroll
          for (int i = 0; i < LE; ++i) acc[q][i] += f[i];
        }
        store_chunk_nt<T>(out + (size_t)t * d + c * LE, acc[q]);
      }
    }
  }
}

// Where a thread owns one chunk and budgets exceed CB, the rows of 16
// assignments are requested together (the sub-expert layer, k <= 32, d = 2048:
// 1.126 -> 1.120 ms per layer in three interleaved pairs, same bits); with
// budgets of at most 8 the wider batch only costs registers (Qwen3-shaped
// layer 0.3 % slower).
template <typename T>
static void launch_combine_t(const T* y, const T* y_shared, const int32_t* tok_off, const float* wts,
                             const int32_t* inv_perm, T* out, int T_, int d, int k_max, hipStream_t st) {
  const int nch = d / (16 / (int)sizeof(T));
  if (nch > 512)
    hipLaunchKernelGGL((combine_kernel<T, 4>), dim3(T_), dim3(256), 0, st, y, y_shared, tok_off, wts, inv_perm, out, d);
  else if (nch > 256)
    hipLaunchKernelGGL((combine_kernel<T, 2>), dim3(T_), dim3(256), 0, st, y, y_shared, tok_off, wts, inv_perm, out, d);
  else if (k_max > CB)
    hipLaunchKernelGGL((combine_kernel<T, 1, 16>), dim3(T_), dim3(256), 0, st, y, y_shared, tok_off, wts, inv_perm, out, d);
  else
    hipLaunchKernelGGL((combine_kernel<T, 1>), dim3(T_), dim3(256), 0, st, y, y_shared, tok_off, wts, inv_perm, out, d);
}

hipError_t launch_combine(int dtype, const void* y, const void* y_shared, const int32_t* tok_off,
                          const float* wts, const int32_t* inv_perm, void* out, int T, int d, int k_max,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (dtype == DT_BF16)
    launch_combine_t<bf16_t>((const bf16_t*)y, (const bf16_t*)y_shared, tok_off, wts, inv_perm, (bf16_t*)out, T, d, k_max, st);
  else
    launch_combine_t<float>((const float*)y, (const float*)y_shared, tok_off, wts, inv_perm, (float*)out, T, d, k_max, st);
  return hipGetLastError();
}

}  // namespace moe
