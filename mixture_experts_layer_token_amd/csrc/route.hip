// Router of the MoE layer: token offsets, router logits and per-token top-k.
//
// Per-request budgets (MoE-Prism, arXiv 2510.19366, §III-C1) arrive as one
// k_t per token.  Selection orders experts by router probability (§III-B2),
// i.e. by logit, ties to the lower index; the weights are the softmax
// renormalised over the selected set, times the routed scaling factor.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace moe {

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Router logits l[t][e] = fp32(sum_i x[t][i] * w[e][i] + b[e]), the sum taken in
// float64 (exact products; only the accumulation rounds) and rounded once.
// Tile: 64 tokens x RE experts per workgroup (RE = 8, 16 or 64, the smallest
// that holds E, so small expert counts do not pay for padding), K staged
// through LDS 32 elements at a time, already widened to float64.  K is split
// over gridDim.z slices so that small batches still fill the chip; slice s
// writes its float64 partial sums to part[s][t][e], and the top-k kernel adds
// the slices in ascending order (any float64 summation order keeps the
// routing contract: exact products, float64 accumulation, one rounding).
// One more slice index (z = S) holds the token-offset scan in its first
// workgroup, so the scan runs beside the tiles instead of before one of them.
constexpr int RT = 64, RK = 32;
constexpr int FUSED_MAX_T = 1024;

// acc + sum of the products of the 16-byte chunks a (x) and b (w), each
// product exact in float64, added in element order.
template <typename T>
__device__ __forceinline__ double dot16_f64(uint4 a, uint4 b, double acc) {
  const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      acc = fma((double)__uint_as_float(ua[i] << 16), (double)__uint_as_float(ub[i] << 16), acc);
      acc = fma((double)__uint_as_float(ua[i] & 0xffff0000u), (double)__uint_as_float(ub[i] & 0xffff0000u), acc);
    } else {
      acc = fma((double)__uint_as_float(ua[i]), (double)__uint_as_float(ub[i]), acc);
    }
  }
  return acc;
}

// NR rows x RK elements of src (rows past nrows read as zero) into dst[k][row].
template <int NR, int LD, typename T>
__device__ __forceinline__ void stage_rows_f64(double (*dst)[LD], const T* __restrict__ src, int row0, int nrows,
                                               int ld, int k0, int tid) {
  constexpr int LE = 16 / sizeof(T);       // elements per 16-byte load
  constexpr int CH = RK / LE;              // loads per row
  constexpr int PER = (NR * CH + 255) / 256;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = tid + 256 * p;
    if (q < NR * CH) {
      const int r = q % NR, c = q / NR;
      uint4 v = zero_u4();
      if (row0 + r < nrows) v = *reinterpret_cast<const uint4*>(src + (size_t)(row0 + r) * ld + k0 + c * LE);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[c * 8 + 2 * i][r] = (double)__uint_as_float(u[i] << 16);
          dst[c * 8 + 2 * i + 1][r] = (double)__uint_as_float(u[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[c * 4 + i][r] = (double)__uint_as_float(u[i]);
      }
    }
  }
}

template <typename T, int RE>
__global__ __launch_bounds__(256) void router_partial_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                             int T_, int d, int E, double* __restrict__ part,
                                                             const int32_t* __restrict__ k, int k_max,
                                                             BudgetPolicy pol, int32_t* __restrict__ tok_off,
                                                             int32_t* __restrict__ status) {
  constexpr int TX = RE < 16 ? RE : 16, EPT = RE / TX, TY = 256 / TX, TPT = RT / TY;
  __shared__ double xs[RK][RT + 1];
  __shared__ double ws[RK][RE + 1];
  __shared__ int32_t scan_part[257];
  const int tid = threadIdx.x;
  const int S = gridDim.z - 1, chunks = d / RK;
  if (blockIdx.z == S) {
    if (blockIdx.x == 0 && blockIdx.y == 0)
      token_offsets_block<256>(k, T_, k_max, pol, tok_off, status, scan_part, scan_part + 256);
    return;
  }
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;
  const int c_beg = (int)(((long long)blockIdx.z * chunks) / S);
  const int c_end = (int)(((long long)(blockIdx.z + 1) * chunks) / S);
  const int ty = tid / TX, tx = tid % TX;
  double acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0;

  for (int c = c_beg; c < c_end; ++c) {
    const int k0 = c * RK;
    stage_rows_f64<RT, RT + 1, T>(xs, x, t0, T_, d, k0, tid);
    stage_rows_f64<RE, RE + 1, T>(ws, w, e0, E, d, k0, tid);
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RK; ++kk) {
      double a[TPT], b[EPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) a[i] = xs[kk][ty + TY * i];
#pragma unroll
      for (int j = 0; j < EPT; ++j) b[j] = ws[kk][tx + TX * j];
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < EPT; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* out = part + (size_t)blockIdx.z * T_ * E;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = t0 + ty + TY * i;
    if (t >= T_) continue;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = e0 + tx + TX * j;
      if (e < E) out[(size_t)t * E + e] = acc[i][j];
    }
  }
}

static int router_tile_e(int E) { return E <= 8 ? 8 : (E <= 16 ? 16 : 64); }

// ---------------------------------------------------------------------------
// Top-k_t per token, one wave64 per token: the S slices of float64 partial
// sums are added in ascending slice order, the bias is added and the sum is
// rounded once to float32; the selection and weights follow select.h.
template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(const double* __restrict__ part, int S,
                                                   const float* __restrict__ bias,
                                                   const int32_t* __restrict__ tok_off, int T_, int E,
                                                   float scale, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, int scratch_slots) {
  extern __shared__ uint64_t topk_scratch[];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  // the partial sums do not depend on the budget: read them before it arrives
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  // G slices of every slot in flight at a time (G * KPL <= 32 loads); each
  // slot's slices are added in ascending order
  constexpr int G = 32 / KPL;
  const size_t qstride = (size_t)T_ * E;
  double acc[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) acc[s] = 0.0;
  for (int q0 = 0; q0 < S; q0 += G) {
    double v[KPL][G];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const int e = lane + 64 * s;
      const double* pe = part + (size_t)t * E + (e < E ? e : 0);
#pragma unroll
      for (int i = 0; i < G; ++i) v[s][i] = (q0 + i < S) ? pe[(size_t)(q0 + i) * qstride] : 0.0;
    }
#pragma unroll
    for (int s = 0; s < KPL; ++s)
#pragma unroll
      for (int i = 0; i < G; ++i) acc[s] += v[s][i];
  }
  uint32_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    key[s] = 0;
    if (e < E) {
      double l = acc[s];
      if (bias) l += (double)bias[e];
      key[s] = logit_key((float)l);
    }
  }
  if (kt == 0) return;
  wave_topk_softmax<KPL>(key, kt, scale, ids + base, wts + base,
                         topk_scratch + (threadIdx.x >> 6) * scratch_slots);
}

// ---------------------------------------------------------------------------
// Fused router for small batches: one workgroup per token sums every logit of
// its token over the whole d in float64 and selects, in one launch.  Each
// workgroup first runs the budget scan of the whole batch (at most
// FUSED_MAX_T budgets) into LDS, so no second launch has to wait for the
// offsets; the first workgroup also writes tok_off and the status.  Thread
// (e, s) of the 256 sums expert e over the 16-byte chunks s, s + S, ... of d
// (EP = E rounded up to a power of two, S = 256 / EP slices), and the slice
// sums of an expert are added in ascending slice order, so the float64
// summation order is fixed.
int fused_router_ok(int T, int d, int E) { return T <= FUSED_MAX_T && E <= 256 && (long long)E * d <= (1 << 19); }
// AUTO takes it only where one workgroup's router rows are few: every
// workgroup streams all E * d router weights, so the Qwen3-shaped layer
// (E * d = 2^18) routes faster split over K (139 vs 155 us per layer), the
// Mixtral-shaped one (2^15) faster fused.
int fused_router_auto(int T, int d, int E) { return fused_router_ok(T, d, E) && (long long)E * d <= (1 << 16); }

template <typename T, int KPL>
__global__ __launch_bounds__(256) void router_fused_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           const int32_t* __restrict__ k, int T_, int d, int E,
                                                           int EP, int k_max, BudgetPolicy pol, float scale,
                                                           int32_t* __restrict__ tok_off, int32_t* __restrict__ status,
                                                           int32_t* __restrict__ ids, float* __restrict__ wts) {
  constexpr int LE = 16 / sizeof(T);
  __shared__ int32_t offs[FUSED_MAX_T + 1];
  __shared__ int32_t scan_part[257];
  __shared__ double red[256];
  __shared__ uint64_t scratch[257];
  const int tid = threadIdx.x, t = blockIdx.x;
  token_offsets_block<256>(k, T_, k_max, pol, offs, t == 0 ? status : nullptr, scan_part, scan_part + 256);
  __syncthreads();
  if (t == 0)
    for (int i = tid; i <= T_; i += 256) tok_off[i] = offs[i];
  if (t >= T_) return;
  const int base = offs[t], kt = offs[t + 1] - base;

  const int S = 256 / EP, e = tid % EP, sl = tid / EP;
  const int nch = d / LE;
  double acc = 0.0;
  if (e < E) {
    const T* xr = x + (size_t)t * d;
    const T* wr = w + (size_t)e * d;
    // eight chunks in flight per thread, added in ascending chunk order
    constexpr int U = 8;
    for (int c0 = sl; c0 < nch; c0 += U * S) {
      uint4 xa[U], wa[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * S;
        xa[u] = c < nch ? *reinterpret_cast<const uint4*>(xr + c * LE) : zero_u4();
        wa[u] = c < nch ? *reinterpret_cast<const uint4*>(wr + c * LE) : zero_u4();
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * S < nch) acc = dot16_f64<T>(xa[u], wa[u], acc);
    }
  }
  red[sl * EP + e] = acc;
  __syncthreads();
  if (tid >= 64 || kt == 0) return;
  const int lane = tid;
  uint32_t key[KPL];
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int ee = lane + 64 * q;
    key[q] = 0;
    if (ee < E) {
      double l = 0.0;
      for (int s2 = 0; s2 < S; ++s2) l += red[s2 * EP + ee];
      if (bias) l += (double)bias[ee];
      key[q] = logit_key((float)l);
    }
  }
  wave_topk_softmax<KPL>(key, kt, scale, ids + base, wts + base, scratch);
}

hipError_t launch_router_fused(int dtype, const void* x, const void* w, const float* bias, const int32_t* k, int T,
                               int d, int E, int k_max, BudgetPolicy pol, float scale, int32_t* tok_off,
                               int32_t* status, int32_t* ids, float* wts, hipStream_t st) {
  if (!fused_router_ok(T, d, E)) return hipErrorInvalidValue;
  int EP = 1;
  while (EP < E) EP *= 2;
  const dim3 grid(max(T, 1));
#define MOE_FUSED(TY, KPL)                                                                                       \
  hipLaunchKernelGGL((router_fused_kernel<TY, KPL>), grid, dim3(256), 0, st, (const TY*)x, (const TY*)w, bias, k, T, \
                     d, E, EP, k_max, pol, scale, tok_off, status, ids, wts)
  if (dtype == DT_BF16) {
    if (E <= 64) MOE_FUSED(bf16_t, 1);
    else if (E <= 128) MOE_FUSED(bf16_t, 2);
    else MOE_FUSED(bf16_t, 4);
  } else {
    if (E <= 64) MOE_FUSED(float, 1);
    else if (E <= 128) MOE_FUSED(float, 2);
    else MOE_FUSED(float, 4);
  }
#undef MOE_FUSED
  return hipGetLastError();
}

int router_splits(int T, int d, int E) {
  if (T == 0) return 1;
  const int tiles = ((T + RT - 1) / RT) * ((E + router_tile_e(E) - 1) / router_tile_e(E));
  const int want = (256 + tiles - 1) / tiles;
  return max(1, min(min(want, 32), d / RK));
}

template <typename T>
static void launch_router_t(const T* x, const T* w, const int32_t* k, int T_, int d, int E, int k_max,
                            BudgetPolicy pol, int S, double* part, int32_t* tok_off, int32_t* status,
                            hipStream_t st) {
  const int RE = router_tile_e(E);
  dim3 grid(max(1, (T_ + RT - 1) / RT), (E + RE - 1) / RE, S + 1);  // slice S: the token scan
  if (RE == 8)
    hipLaunchKernelGGL((router_partial_kernel<T, 8>), grid, dim3(256), 0, st, x, w, T_, d, E, part, k, k_max, pol,
                       tok_off, status);
  else if (RE == 16)
    hipLaunchKernelGGL((router_partial_kernel<T, 16>), grid, dim3(256), 0, st, x, w, T_, d, E, part, k, k_max, pol,
                       tok_off, status);
  else
    hipLaunchKernelGGL((router_partial_kernel<T, 64>), grid, dim3(256), 0, st, x, w, T_, d, E, part, k, k_max, pol,
                       tok_off, status);
}

hipError_t launch_router(int dtype, const void* x, const void* w, const int32_t* k, int T, int d, int E, int k_max,
                         BudgetPolicy pol, int S, double* part, int32_t* tok_off, int32_t* status, hipStream_t st) {
  if (dtype == DT_BF16)
    launch_router_t<bf16_t>((const bf16_t*)x, (const bf16_t*)w, k, T, d, E, k_max, pol, S, part, tok_off, status, st);
  else
    launch_router_t<float>((const float*)x, (const float*)w, k, T, d, E, k_max, pol, S, part, tok_off, status, st);
  return hipGetLastError();
}

hipError_t launch_topk(const double* part, int S, const float* bias, const int32_t* tok_off, int T, int E,
                       int k_max, float scale, int32_t* ids, float* wts, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4);
  const int slots = k_max + 1;
  const size_t lds = (size_t)4 * slots * sizeof(uint64_t);
#define MOE_TOPK(KPL) \
  hipLaunchKernelGGL(topk_kernel<KPL>, grid, dim3(256), lds, st, part, S, bias, tok_off, T, E, scale, ids, wts, slots)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
