// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// bfloat16 is carried as raw 16-bit storage everywhere outside MFMA operands.
typedef uint16_t bf16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16 bytes in registers (native vector)

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elt<bf16_t> {
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// One 16x16 MFMA tile step.  EPV = elements of K each lane supplies per
// instruction; a 16-byte load holds LOAD_ELEMS elements.
//  bf16: v_mfma_f32_16x16x32_bf16 (8 K-elements per lane, 32 per instruction)
//  fp32: v_mfma_f32_16x16x4_f32   (1 K-element per lane, 4 per instruction)
// A operand: lane l supplies row (l % 16); B operand: column (l % 16); both
// supply the same K indices, chosen by lane group (l / 16).  The 16x16 f32
// result holds D[4 * (l / 16) + r][l % 16] in element r of lane l.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int EPV = 8;
  static constexpr int LOAD_ELEMS = 8;
  __device__ __forceinline__ static f32x4_t step(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t step(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int EPV = 1;
  static constexpr int LOAD_ELEMS = 4;
};

__device__ __forceinline__ f32x4_t mfma_f32_4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Inclusive prefix sum of one int per thread over a workgroup of NT threads
// (a multiple of 64): a shuffle scan inside each wave, then the totals of the
// lower waves.  `wsum` is NT / 64 ints of LDS; the trailing barrier lets the
// caller reuse it at once.
template <int NT>
__device__ __forceinline__ int block_scan_incl(int v, int32_t* wsum) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) add += i < w ? wsum[i] : 0;
  __syncthreads();
  return v + add;
}

// Maximum of one int per thread over a workgroup of NT threads (a multiple of
// 64); `wsum` is NT / 64 ints of LDS; every thread gets the result.
template <int NT>
__device__ __forceinline__ int block_max(int v, int32_t* wsum) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  int m = wsum[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = max(m, wsum[i]);
  __syncthreads();
  return m;
}

// ---- global->LDS DMA and explicit waits ----
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N> __device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}
// vm_wait<n> for a wave-uniform n in [0, NMAX] (the count must be an immediate).
template <int NMAX> __device__ __forceinline__ void vm_wait_dyn(int n) {
  if constexpr (NMAX <= 0) {
    vm_wait<0>();
  } else {
    if (n >= NMAX) vm_wait<NMAX>();
    else vm_wait_dyn<NMAX - 1>(n);
  }
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// LDS tiles of 128-byte rows: the eight 16-byte chunks of row r are
// XOR-permuted by (r >> 1) & 7, which keeps both 16-row x 16-byte and
// 32-row x 32-byte fragment reads free of bank conflicts.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
// byte offset of 16-byte chunk c of tile row r
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ lds_swz(r)) * 16); }

// ---- expert weight storage (moe_weight_layout) ----
// Row-major: element (n, k) of a [N][K] matrix at n * K + k.  Blocked: the
// matrix is cut into 64-row x 128-byte blocks (EB = 128 / sizeof(T)
// elements of K), block (n / 64, k / EB) at (n / 64 * (K / EB) + k / EB) *
// 64 * EB, rows of a block contiguous.  With both, every 16-byte chunk that
// starts at a multiple of 16 bytes of a row is contiguous, and a run of K
// that stays inside one EB-aligned step advances by 1 per element.
template <typename T>
__host__ __device__ __forceinline__ size_t w_offset(int n, int k, int K, int blocked) {
  constexpr int EB = 128 / (int)sizeof(T);
  if (!blocked) return (size_t)n * K + k;
  return ((size_t)(n >> 6) * (K / EB) + k / EB) * (64 * EB) + (size_t)(n & 63) * EB + (k % EB);
}
// Elements between the same (row, k % EB) position of two consecutive
// EB-wide steps of K.
template <typename T>
__host__ __device__ __forceinline__ int w_kstep(int blocked) {
  constexpr int EB = 128 / (int)sizeof(T);
  return blocked ? 64 * EB : EB;
}
// Elements between rows n and n + dn inside one 64-row block (blocked), or
// anywhere (row-major).
template <typename T>
__host__ __device__ __forceinline__ size_t w_rowstep(int dn, int K, int blocked) {
  constexpr int EB = 128 / (int)sizeof(T);
  return blocked ? (size_t)dn * EB : (size_t)dn * K;
}

}  // namespace moe
