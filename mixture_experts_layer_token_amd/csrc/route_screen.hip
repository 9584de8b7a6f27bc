// Screened router for large bf16 batches: bf16 MFMA logits with a proven error
// bound pick the few candidates whose exact logit can matter, and only those
// get the float64 dot product of the routing contract.
//
// The contract (shared with the plain router): l[t][e] = fp32(sum_i x_i w_i + b_e)
// with the sum accumulated in float64 from exact products; experts ordered by
// (l descending, e ascending).  The screen never changes which experts are
// selected, their order or their weights -- it only avoids computing exact
// logits that cannot enter the top-k_t.
//
// Pass 1 (MFMA): a[t][e] = sum x_i w_i and s[t][e] = sum |x_i||w_i| in fp32 with
// v_mfma_f32_16x16x32_bf16.  Products of bf16 values are exact in fp32, so in
// any summation order |a - exact| <= d * u * S with u = 2^-24 (2^-23 if the
// hardware truncates) and S <= s / (1 - d u).  The radius used is
// r = d * 2^-22 * s (+ a tiny floor), which covers both.
//
// Pass 2 (one wave per token): lower_e = a + b - r, upper_e = a + b + r (fp64).
// L = k_t-th largest lower bound.  Expert e is a candidate iff
// upper_e >= L - m, m = 2^-21 |L| + 2^-126 (four fp32 ulps at L).  A
// non-candidate is beaten by k_t experts whose exact logits exceed its own by
// more than m, so their fp32 logits are strictly larger: it cannot be selected.
// Candidates get the exact fp64 dot product; the usual wave top-k runs on their
// exact fp32 logits (non-candidates are never reached, since the k_t experts
// defining L are candidates).
#include "common.h"
#include "launch.h"

namespace moe {

// ---- pass 1: approximate logits and |x||w| sums, 64 tokens x 64 experts per WG
// 4 waves in 2 x 2, each 32 experts x 32 tokens = 2 x 2 tiles of 16 x 16.
__global__ __launch_bounds__(256) void router_screen_mfma_kernel(const bf16_t* __restrict__ x,
                                                                 const bf16_t* __restrict__ w, int T, int d, int E,
                                                                 float* __restrict__ approx, float* __restrict__ absum) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int e0 = blockIdx.y * 64 + (wave >> 1) * 32;
  // operand rows (clamped in range; results of clamped rows are not stored)
  const bf16_t* wr[2];
  const bf16_t* xr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    wr[i] = w + (size_t)min(e0 + i * 16 + lr, E - 1) * d + lg * 8;
    xr[i] = x + (size_t)min(t0 + i * 16 + lr, T - 1) * d + lg * 8;
  }
  f32x4_t acc[2][2], aab[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      aab[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  const u32x4_t sign_off = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
  u32x4_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = *reinterpret_cast<const u32x4_t*>(wr[i]);
    b[i] = *reinterpret_cast<const u32x4_t*>(xr[i]);
  }
  for (int k = 0; k < d; k += 32) {
    const int kn = (k + 32 < d) ? k + 32 : k;  // next step (the last re-reads, cached)
    u32x4_t na[2], nb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      na[i] = *reinterpret_cast<const u32x4_t*>(wr[i] + kn);
      nb[i] = *reinterpret_cast<const u32x4_t*>(xr[i] + kn);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = Mfma<bf16_t>::step(a[i], b[j], acc[i][j]);
        aab[i][j] = Mfma<bf16_t>::step(a[i] & sign_off, b[j] & sign_off, aab[i][j]);
      }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = na[i];
      b[i] = nb[i];
    }
  }
  // lane holds D[e = 4*lg + r][t = lr] of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = t0 + j * 16 + lr;
      if (t >= T) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + i * 16 + 4 * lg + r;
        if (e < E) {
          approx[(size_t)t * E + e] = acc[i][j][r];
          absum[(size_t)t * E + e] = aab[i][j][r];
        }
      }
    }
}

__device__ __forceinline__ uint64_t dkey(double v) {  // order-preserving image of a double
  uint64_t u = __double_as_longlong(v);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t wave_max_u64s(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// exact fp64 dots of one token row with NC expert rows (bf16), the whole wave
// cooperating: lane l takes elements [8l + 512i, +8); results are wave sums.
template <int NC>
__device__ __forceinline__ void exact_dots(const bf16_t* __restrict__ xr, const bf16_t* const (&wr)[NC], int d,
                                           int lane, double (&out)[NC]) {
  double acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.0;
  for (int i = lane * 8; i < d; i += 512) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + i);
    uint4 wv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) wv[c] = *reinterpret_cast<const uint4*>(wr[c] + i);
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
    double xd[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xd[2 * q] = (double)__uint_as_float(xs[q] << 16);
      xd[2 * q + 1] = (double)__uint_as_float(xs[q] & 0xffff0000u);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t ws[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[c] = fma(xd[2 * q], (double)__uint_as_float(ws[q] << 16), acc[c]);
        acc[c] = fma(xd[2 * q + 1], (double)__uint_as_float(ws[q] & 0xffff0000u), acc[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) out[c] = wave_sum_f64(acc[c]);
}

// ---- pass 2: candidates, exact logits, top-k_t and weights; one wave per token
template <int KPL>
__global__ __launch_bounds__(256) void router_screen_select_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ approx, const float* __restrict__ absum, const int32_t* __restrict__ tok_off, int T,
    int d, int E, float scale, int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  if (kt == 0) return;
  const double rad_scale = (double)d * 0x1p-22;
  double lower[KPL], upper[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    lower[s] = -INFINITY;
    upper[s] = -INFINITY;
    if (e < E) {
      const double c = (double)approx[(size_t)t * E + e] + (bias ? (double)bias[e] : 0.0);
      const double r = rad_scale * (double)absum[(size_t)t * E + e] + 0x1p-126;
      lower[s] = c - r;
      upper[s] = c + r;
    }
  }
  // L = kt-th largest lower bound.  Keys: the order-preserving image of the
  // bound with its low 10 bits replaced by the inverted expert index, so keys
  // are unique; the truncation only lowers L (more candidates, still exact).
  uint64_t lk[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    lk[s] = (e < E) ? ((dkey(lower[s]) & ~0x3ffull) | (uint64_t)(1023 - e)) : 0;
  }
  uint64_t kth = 0;
  for (int j = 0; j < kt; ++j) {
    uint64_t m = lk[0];
#pragma unroll
    for (int s = 1; s < KPL; ++s) m = lk[s] > m ? lk[s] : m;
    m = wave_max_u64s(m);
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      if (lk[s] == m) lk[s] = 0;
    kth = m;
  }
  uint64_t ku = kth & ~0x3ffull;
  ku = (ku & 0x8000000000000000ull) ? (ku & 0x7fffffffffffffffull) : ~ku;
  const double L = __longlong_as_double(ku);
  const double cut = L - (fabs(L) * 0x1p-21 + 0x1p-126);

  // candidate list (ascending expert index) in LDS, then exact logits four at a time
  __shared__ int32_t clist_all[4][1024];
  int32_t* clist = clist_all[threadIdx.x >> 6];
  int ncand = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    const bool cand = (e < E) && (upper[s] >= cut);
    const uint64_t mask = __ballot(cand);
    if (cand) clist[ncand + __popcll(mask & ((1ull << lane) - 1ull))] = e;
    ncand += __popcll(mask);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bf16_t* xr = x + (size_t)t * d;
  uint64_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) key[s] = 0;
  for (int c0 = 0; c0 < ncand; c0 += 4) {
    int ce[4];
    const bf16_t* wr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ce[c] = clist[min(c0 + c, ncand - 1)];  // past the end: repeat the last candidate (result unused)
      wr[c] = w + (size_t)ce[c] * d;
    }
    double v[4];
    exact_dots<4>(xr, wr, d, lane, v);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c0 + c >= ncand) continue;
      double vv = v[c];
      if (bias) vv += (double)bias[ce[c]];
      float l = (float)vv;
      if (l == 0.0f) l = 0.0f;
      uint32_t u = __float_as_uint(l);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const uint64_t kk = (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(0xffffffffu - (uint32_t)ce[c]);
      if (lane == (ce[c] & 63)) {
#pragma unroll
        for (int s = 0; s < KPL; ++s)
          if ((ce[c] >> 6) == s) key[s] = kk;
      }
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
    m = wave_max_u64s(m);
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

hipError_t launch_router_screen(const void* x, const void* w, const float* bias, const int32_t* tok_off, int T,
                                int d, int E, float scale, float* approx, float* absum, int32_t* ids, float* wts,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_screen_mfma_kernel, dim3((T + 63) / 64, (E + 63) / 64), dim3(256), 0, st,
                     (const bf16_t*)x, (const bf16_t*)w, T, d, E, approx, absum);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 grid((T + 3) / 4);
#define MOE_SEL(KPL)                                                                                            \
  hipLaunchKernelGGL(router_screen_select_kernel<KPL>, grid, dim3(256), 0, st, (const bf16_t*)x, (const bf16_t*)w, \
                     bias, approx, absum, tok_off, T, d, E, scale, ids, wts)
  if (E <= 64) MOE_SEL(1);
  else if (E <= 128) MOE_SEL(2);
  else if (E <= 256) MOE_SEL(4);
  else if (E <= 512) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
