// Router of the MoE layer: token offsets, router logits and per-token top-k.
//
// Per-request budgets (MoE-Prism, arXiv 2510.19366, §III-C1) arrive as one
// k_t per token.  Selection orders experts by router probability (§III-B2),
// i.e. by logit, ties to the lower index; the weights are the softmax
// renormalised over the selected set, times the routed scaling factor.
#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// tok_off = exclusive prefix sum of the validated budgets; one workgroup.
// A k_t outside [0, k_max] counts as 0 and raises MOE_DEV_BAD_K.
__global__ __launch_bounds__(1024) void tok_offsets_kernel(const int32_t* __restrict__ k, int T,
                                                           int k_max, int32_t* __restrict__ tok_off,
                                                           int32_t* __restrict__ status) {
  __shared__ int32_t part[1024];
  __shared__ int32_t bad_any;
  const int tid = threadIdx.x;
  const int per = (T + 1023) / 1024;
  const int beg = min(tid * per, T), end = min(beg + per, T);
  int s = 0, bad = 0;
  for (int i = beg; i < end; ++i) {
    int v = k[i];
    if (v < 0 || v > k_max) { v = 0; bad = 1; }
    s += v;
  }
  if (tid == 0) bad_any = 0;
  part[tid] = s;
  __syncthreads();
  if (bad) atomicOr(&bad_any, 1);
  for (int off = 1; off < 1024; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int i = beg; i < end; ++i) {
    tok_off[i] = run;
    int v = k[i];
    if (v < 0 || v > k_max) v = 0;
    run += v;
  }
  if (tid == 1023) tok_off[T] = part[1023];
  if (tid == 0 && status) status[0] = bad_any ? MOE_DEV_BAD_K_BIT : 0;
}

// ---------------------------------------------------------------------------
// Router logits l[t][e] = fp32(sum_i x[t][i] * w[e][i] + b[e]), the sum taken in
// float64 (exact products; only the accumulation rounds) and rounded once.
// Tile: 64 tokens x 64 experts per workgroup, 4x4 outputs per thread, K staged
// through LDS 32 elements at a time, already widened to float64.
constexpr int RT = 64, RE = 64, RK = 32, RPAD = 65;

template <typename T>
__device__ __forceinline__ void stage_rows_f64(double (*dst)[RPAD], const T* __restrict__ src,
                                               int row0, int nrows, int ld, int k0, int tid);

template <>
__device__ __forceinline__ void stage_rows_f64<bf16_t>(double (*dst)[RPAD], const bf16_t* __restrict__ src,
                                                       int row0, int nrows, int ld, int k0, int tid) {
  // 64 rows x 32 bf16 = 256 chunks of 8 elements; one per thread.
  const int r = tid & 63, c = tid >> 6;
  uint4 v = zero_u4();
  if (row0 + r < nrows) v = *reinterpret_cast<const uint4*>(src + (size_t)(row0 + r) * ld + k0 + c * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[c * 8 + 2 * i][r] = (double)__uint_as_float(w[i] << 16);
    dst[c * 8 + 2 * i + 1][r] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void stage_rows_f64<float>(double (*dst)[RPAD], const float* __restrict__ src,
                                                      int row0, int nrows, int ld, int k0, int tid) {
  // 64 rows x 32 floats = 512 chunks of 4 elements; two per thread.
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p;
    const int r = q & 63, c = q >> 6;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + r < nrows) v = *reinterpret_cast<const float4*>(src + (size_t)(row0 + r) * ld + k0 + c * 4);
    dst[c * 4 + 0][r] = (double)v.x;
    dst[c * 4 + 1][r] = (double)v.y;
    dst[c * 4 + 2][r] = (double)v.z;
    dst[c * 4 + 3][r] = (double)v.w;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void router_logits_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                            const float* __restrict__ bias, int T_, int d, int E,
                                                            float* __restrict__ logits) {
  __shared__ double xs[RK][RPAD];
  __shared__ double ws[RK][RPAD];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;
  const int ty = tid >> 4, tx = tid & 15;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += RK) {
    stage_rows_f64<T>(xs, x, t0, T_, d, k0, tid);
    stage_rows_f64<T>(ws, w, e0, E, d, k0, tid);
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RK; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty + 16 * i;
    if (t >= T_) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e >= E) continue;
      double v = acc[i][j];
      if (bias) v += (double)bias[e];
      logits[(size_t)t * E + e] = (float)v;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k_t per token, one wave64 per token.  Every expert becomes a 64-bit key:
// high word = order-preserving image of the float32 logit (-0 folded to +0),
// low word = ~e, so the largest key is the largest logit with the lowest
// index.  k_t rounds of (lane max, wave max via xor-shuffles, remove winner)
// emit the experts best first.  The softmax over the selected logits is
// accumulated on the fly (every lane sees every winner), so each lane keeps
// only the unnormalised weights of the slots it will write.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const int32_t* __restrict__ tok_off, int T_, int E,
                                                   float scale, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  uint64_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    key[s] = 0;
    if (e < E) {
      float l = logits[(size_t)t * E + e];
      if (l == 0.0f) l = 0.0f;
      uint32_t u = __float_as_uint(l);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[s] = (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(0xffffffffu - (uint32_t)e);
    }
  }
  float mine[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) mine[s] = 0.f;
  float l0 = 0.f, sum = 0.f;
  for (int j = 0; j < kt; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int s = 1; s < KPL; ++s) m = key[s] > m ? key[s] : m;
    m = wave_max_u64(m);
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      if (key[s] == m) key[s] = 0;
    const int e = (int)(0xffffffffu - (uint32_t)(m & 0xffffffffu));
    uint32_t u = (uint32_t)(m >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    const float l = __uint_as_float(u);
    if (j == 0) l0 = l;
    const float p = expf(l - l0);
    sum += p;
    if (lane == (j & 63)) {
#pragma unroll
      for (int s = 0; s < KPL; ++s)
        if ((j >> 6) == s) mine[s] = p;
      ids[base + j] = e;
    }
  }
  const float inv = scale / sum;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int j = lane + 64 * s;
    if (j < kt) wts[base + j] = mine[s] * inv;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_tok_offsets(const int32_t* k, int T, int k_max, int32_t* tok_off, int32_t* status,
                              hipStream_t st) {
  hipLaunchKernelGGL(tok_offsets_kernel, dim3(1), dim3(1024), 0, st, k, T, k_max, tok_off, status);
  return hipGetLastError();
}

hipError_t launch_router_logits(int dtype, const void* x, const void* w, const float* bias, int T, int d,
                                int E, float* logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + RT - 1) / RT, (E + RE - 1) / RE);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(router_logits_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x,
                       (const bf16_t*)w, bias, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, st, (const float*)x,
                       (const float*)w, bias, T, d, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const int32_t* tok_off, int T, int E, float scale, int32_t* ids,
                       float* wts, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  if (E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, st, logits, tok_off, T, E, scale, ids, wts);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, st, logits, tok_off, T, E, scale, ids, wts);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, st, logits, tok_off, T, E, scale, ids, wts);
  else if (E <= 512)
    hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, st, logits, tok_off, T, E, scale, ids, wts);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, st, logits, tok_off, T, E, scale, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
