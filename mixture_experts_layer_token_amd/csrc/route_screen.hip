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
// v_mfma_f32_16x16x32_bf16, K split over S slices (partial sums per slice, added
// in slice order by pass 2).  Products of bf16 values are exact in fp32, so in
// any summation order of depth n the error is at most n * u * S with
// u = 2^-24 (2^-23 if the hardware truncates) and S <= s / (1 - n u); the
// slices make n <= d/S + S <= d.  The radius used is r = d * 2^-22 * s (+ a
// tiny floor), which covers both roundings with a factor of two to spare.
//
// Pass 2 (one wave per token): lower_e = a + b - r, upper_e = a + b + r (fp64).
// L = the k_t-th largest lower bound, each rounded down to fp32 first (a
// smaller L only adds candidates).  Expert e is a candidate iff
// upper_e >= L - m, m = 2^-21 |L| + 2^-126 (four fp32 ulps at L).  A
// non-candidate is beaten by k_t experts whose exact logits exceed its own by
// more than m, so their fp32 logits are strictly larger: it cannot be selected.
// Candidates get the exact fp64 dot product; the top-k of select.h runs on
// their exact fp32 logits (non-candidates are never reached, since the k_t
// experts defining L are candidates).
#include "common.h"
#include "launch.h"
#include "screen.h"
#include "select.h"

namespace moe {

// ---- pass 1: partial approximate logits and |x||w| sums of one K slice.
// A workgroup covers 64 tokens x 256 experts: wave w takes experts
// [64w, 64w + 64) of the span as a 4 x 4 grid of 16 x 16 MFMA tiles.  The four
// waves read the same token rows (hits in the CU's L1 after the first), so the
// bytes fetched per MFMA are a quarter of a one-tile-per-wave split.
// One more slice index (z = S) holds the token-offset scan (pass 2 needs it)
// in its first workgroup; its other workgroups exit at once.  Dispatched after
// the tiles, the scan shares a CU with one of them instead of delaying one.
__global__ __launch_bounds__(256) void router_screen_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int d, int E, float* __restrict__ approx,
    float* __restrict__ absum, const int32_t* __restrict__ k, int k_max, BudgetPolicy pol,
    int32_t* __restrict__ tok_off, int32_t* __restrict__ status) {
  if (blockIdx.z == gridDim.z - 1) {
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      __shared__ int32_t scan_part[257];
      token_offsets_block<256>(k, T, k_max, pol, tok_off, status, scan_part, scan_part + 256);
    }
    return;
  }
  if (T == 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * 256 + wave * 64;
  if (e0 >= E) return;
  const int S = gridDim.z - 1, chunks = d / 32;
  const int k_beg = (int)(((long long)blockIdx.z * chunks) / S) * 32;
  const int k_end = (int)(((long long)(blockIdx.z + 1) * chunks) / S) * 32;
  // operand rows (clamped in range; results of clamped rows are not stored)
  const bf16_t* wr[4];
  const bf16_t* xr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wr[i] = w + (size_t)min(e0 + i * 16 + lr, E - 1) * d + lg * 8;
    xr[i] = x + (size_t)min(t0 + i * 16 + lr, T - 1) * d + lg * 8;
  }
  f32x4_t acc[4][4], aab[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      aab[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  const u32x4_t sign_off = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
  if (k_beg < k_end) {
    u32x4_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const u32x4_t*>(wr[i] + k_beg);
      b[i] = *reinterpret_cast<const u32x4_t*>(xr[i] + k_beg);
    }
    for (int kk = k_beg; kk < k_end; kk += 32) {
      const int kn = (kk + 32 < k_end) ? kk + 32 : kk;  // next step (the last re-reads, cached)
      u32x4_t na[4], nb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        na[i] = *reinterpret_cast<const u32x4_t*>(wr[i] + kn);
        nb[i] = *reinterpret_cast<const u32x4_t*>(xr[i] + kn);
      }
      u32x4_t aa[4], ab[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aa[i] = a[i] & sign_off;
        ab[i] = b[i] & sign_off;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = Mfma<bf16_t>::step(a[i], b[j], acc[i][j]);
          aab[i][j] = Mfma<bf16_t>::step(aa[i], ab[j], aab[i][j]);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = na[i];
        b[i] = nb[i];
      }
    }
  }
  // lane holds D[e = 4*lg + r][t = lr] of each tile
  float* const ap = approx + (size_t)blockIdx.z * T * E;
  float* const sp = absum + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + j * 16 + lr;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + i * 16 + 4 * lg;
      if ((E & 3) == 0 && e + 3 < E) {
        *reinterpret_cast<float4*>(ap + (size_t)t * E + e) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<float4*>(sp + (size_t)t * E + e) = make_float4(aab[i][j][0], aab[i][j][1], aab[i][j][2], aab[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < E) {
            ap[(size_t)t * E + e + r] = acc[i][j][r];
            sp[(size_t)t * E + e + r] = aab[i][j][r];
          }
      }
    }
  }
}

// ---- pass 2: candidates, exact logits, top-k_t and weights; one wave per token.
// XR: the token row fits one pass (d <= 512 * XC) and is loaded once, before
// the candidates, instead of once per candidate.
template <int KPL, int XC, bool XR>
__global__ __launch_bounds__(256) void router_screen_select_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ approx, const float* __restrict__ absum, int S, const int32_t* __restrict__ tok_off,
    int T, int d, int E, float scale, int32_t* __restrict__ ids, float* __restrict__ wts, int red_words,
    int lds_words) {
  extern __shared__ uint64_t sel_lds[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  // the slice partials do not depend on the budget: read them before it arrives
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  // per-wave LDS: [red_words: lane shares of SEL_GRP candidates, later the
  // top-k scratch][E int32: candidate list][E doubles: exact sums by candidate]
  uint64_t* const area = sel_lds + (size_t)wv * lds_words;
  double* const red = reinterpret_cast<double*>(area);
  int32_t* const clist = reinterpret_cast<int32_t*>(area + red_words);
  double* const cval = reinterpret_cast<double*>(area + red_words + (E + 1) / 2);

  // bounds from the slice partials (added in slice order); the bias of the
  // lane's experts stays in registers
  const double rad_scale = (double)d * 0x1p-22;
  double cen[KPL], rad[KPL];
  float bs[KPL];
  uint32_t lkey[KPL];
  const size_t sstride = (size_t)T * E;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    cen[s] = 0.0;
    rad[s] = 0.0;
    lkey[s] = 0;
    bs[s] = 0.f;
    if (e < E) {
      if (bias) bs[s] = bias[e];
      // slices in ascending order, eight loads in flight at a time
      float a = 0.f, m = 0.f;
      const float* pa = approx + (size_t)t * E + e;
      const float* pm = absum + (size_t)t * E + e;
      for (int q0 = 0; q0 < S; q0 += 8) {
        float va[8], vm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          va[i] = (q0 + i < S) ? pa[(size_t)(q0 + i) * sstride] : 0.f;
          vm[i] = (q0 + i < S) ? pm[(size_t)(q0 + i) * sstride] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a += va[i];
          m += vm[i];
        }
      }
      cen[s] = (double)a + (double)bs[s];
      rad[s] = rad_scale * (double)m + 0x1p-126;
      lkey[s] = logit_key(__double2float_rd(cen[s] - rad[s]));
    }
  }
  if (kt == 0) return;
  const float L = key_logit(wave_kth_largest<KPL>(lkey, kt));
  const double cut = (double)L - (fabs((double)L) * 0x1p-21 + 0x1p-126);

  // candidate list, ascending expert index; cidx = a slot's place in it
  int ncand = 0;
  int cidx[KPL];
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int e = lane + 64 * s;
    const bool cand = (e < E) && (cen[s] + rad[s] >= cut);
    const uint64_t mask = __ballot(cand);
    cidx[s] = cand ? ncand + __popcll(mask & below) : -1;
    if (cand) clist[cidx[s]] = e;
    ncand += __popcll(mask);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // exact logits of the candidates
  exact_dots<XC, XR, SEL_GRP, XR ? 4 : 2>(
      x + (size_t)t * d, d, ncand, [&](int c) { return w + (size_t)clist[c] * d; }, red,
      [&](int c, double v) { cval[c] = v; });
  // keys of the candidates (bias added in float64 before the one rounding)
  uint32_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) key[s] = cidx[s] >= 0 ? logit_key((float)(cval[cidx[s]] + (double)bs[s])) : 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  wave_topk_softmax<KPL>(key, kt, scale, ids + base, wts + base, area);
}

// ---- pass 2 for a wide hidden size: one workgroup of four waves per token.
// Wave 0 takes the bounds and the candidate list as above; then every wave
// takes a quarter of d, keeps that slice of the token row in registers (as
// bf16: widened to float64 it held 32 more registers and one workgroup fewer
// per CU, 120 against 102 us on 4,096 tokens, d = 7168, same bits) and sums
// the candidates' exact partial dots over it with DEPTH candidates' weight
// chunks in flight, so that the token row is read once instead of once per
// candidate; wave 0 adds the four partials in wave order (float64), adds the
// bias, rounds once and selects.  XCS: 512-element chunks per wave slice
// (d / 4 <= 512 * XCS).
template <int KPL, int XCS, int DEPTH>
__global__ __launch_bounds__(256) void router_screen_select_wg_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ approx, const float* __restrict__ absum, int S, const int32_t* __restrict__ tok_off,
    int T, int d, int E, float scale, int32_t* __restrict__ ids, float* __restrict__ wts, int red_words) {
  extern __shared__ uint64_t sel_lds[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x;
  // LDS: [4][red_words: lane shares of SEL_GRP candidates; wave 0's later the
  // top-k scratch][4][E doubles: partial sums by candidate][E int32: candidate
  // list][1 int32: candidate count]
  double* const red = reinterpret_cast<double*>(sel_lds + (size_t)wv * red_words);
  double* const part = reinterpret_cast<double*>(sel_lds + (size_t)4 * red_words);
  int32_t* const clist = reinterpret_cast<int32_t*>(sel_lds + (size_t)4 * red_words + (size_t)4 * E);
  int32_t* const ncand_l = clist + E;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;

  double cen[KPL], rad[KPL];
  float bs[KPL];
  int cidx[KPL];
  if (wv == 0) {
    const double rad_scale = (double)d * 0x1p-22;
    uint32_t lkey[KPL];
    const size_t sstride = (size_t)T * E;
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const int e = lane + 64 * s;
      cen[s] = 0.0;
      rad[s] = 0.0;
      lkey[s] = 0;
      bs[s] = 0.f;
      if (e < E) {
        if (bias) bs[s] = bias[e];
        float a = 0.f, m = 0.f;
        const float* pa = approx + (size_t)t * E + e;
        const float* pm = absum + (size_t)t * E + e;
        for (int q0 = 0; q0 < S; q0 += 8) {
          float va[8], vm[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            va[i] = (q0 + i < S) ? pa[(size_t)(q0 + i) * sstride] : 0.f;
            vm[i] = (q0 + i < S) ? pm[(size_t)(q0 + i) * sstride] : 0.f;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            a += va[i];
            m += vm[i];
          }
        }
        cen[s] = (double)a + (double)bs[s];
        rad[s] = rad_scale * (double)m + 0x1p-126;
        lkey[s] = logit_key(__double2float_rd(cen[s] - rad[s]));
      }
    }
    int ncand = 0;
#pragma unroll
    for (int s = 0; s < KPL; ++s) cidx[s] = -1;
    if (kt > 0) {
      const float L = key_logit(wave_kth_largest<KPL>(lkey, kt));
      const double cut = (double)L - (fabs((double)L) * 0x1p-21 + 0x1p-126);
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int s = 0; s < KPL; ++s) {
        const int e = lane + 64 * s;
        const bool cand = (e < E) && (cen[s] + rad[s] >= cut);
        const uint64_t mask = __ballot(cand);
        cidx[s] = cand ? ncand + __popcll(mask & below) : -1;
        if (cand) clist[cidx[s]] = e;
        ncand += __popcll(mask);
      }
    }
    if (lane == 0) *ncand_l = ncand;
  }
  __syncthreads();
  const int ncand = *ncand_l;
  // this wave's slice of the exact dots
  const int dq = d / 4, k0 = wv * dq;
  double* const mine = part + (size_t)wv * E;
  exact_dots<XCS, true, SEL_GRP, DEPTH, true>(
      x + (size_t)t * d + k0, dq, ncand, [&](int c) { return w + (size_t)clist[c] * d + k0; }, red,
      [&](int c, double v) { mine[c] = v; });
  __syncthreads();
  if (wv != 0 || kt == 0) return;
  uint32_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    key[s] = 0u;
    if (cidx[s] >= 0) {
      const int c = cidx[s];
      const double v = ((part[c] + part[E + c]) + part[2 * E + c]) + part[3 * E + c];
      key[s] = logit_key((float)(v + (double)bs[s]));
    }
  }
  wave_topk_softmax<KPL>(key, kt, scale, ids + base, wts + base, sel_lds);
}

// Slices: enough workgroups (64 tokens x 256 experts each) to give every CU
// one, at least two 32-element steps per slice, and at most 2^22 partial
// entries per array.
int router_screen_splits(int T, int d, int E) {
  const long long wgs = (long long)max(1, (T + 63) / 64) * ((E + 255) / 256);
  long long S = (256 + wgs - 1) / wgs;
  S = min(S, (long long)max(1, d / 64));
  S = min(S, 32LL);
  S = min(S, max(1LL, (4LL << 20) / max(1LL, (long long)T * E)));
  return (int)max(1LL, S);
}

template <int KPL, int XC>
static void launch_select(dim3 grid, size_t lds, hipStream_t st, const bf16_t* x, const bf16_t* w, const float* bias,
                          const float* approx, const float* absum, int S, const int32_t* tok_off, int T, int d, int E,
                          float scale, int32_t* ids, float* wts, int red_words, int words) {
  if (d <= 512 * XC)
    hipLaunchKernelGGL((router_screen_select_kernel<KPL, XC, true>), grid, dim3(256), lds, st, x, w, bias, approx,
                       absum, S, tok_off, T, d, E, scale, ids, wts, red_words, words);
  else
    hipLaunchKernelGGL((router_screen_select_kernel<KPL, XC, false>), grid, dim3(256), lds, st, x, w, bias, approx,
                       absum, S, tok_off, T, d, E, scale, ids, wts, red_words, words);
}

hipError_t launch_router_screen_partials(const void* x, const void* w, const int32_t* k, int T, int d, int E,
                                         int k_max, BudgetPolicy pol, int S, float* approx, float* absum,
                                         int32_t* tok_off, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(router_screen_mfma_kernel, dim3(max(1, (T + 63) / 64), (E + 255) / 256, S + 1), dim3(256), 0, st,
                     (const bf16_t*)x, (const bf16_t*)w, T, d, E, approx, absum, k, k_max, pol, tok_off, status);
  return hipGetLastError();
}

hipError_t launch_router_screen(const void* x, const void* w, const float* bias, const int32_t* k, int T, int d,
                                int E, int k_max, BudgetPolicy pol, int S, float scale, float* approx, float* absum,
                                int32_t* tok_off, int32_t* status, int32_t* ids, float* wts, hipStream_t st) {
  hipError_t err = launch_router_screen_partials(x, w, k, T, d, E, k_max, pol, S, approx, absum, tok_off, status, st);
  if (err != hipSuccess || T == 0) return err;
  if (d >= 4096 && d <= 8192) {
    // wide rows: a workgroup per token, the row split over its four waves
    const int red_words = max(SEL_GRP * 64, k_max + 1);
    const size_t lds = ((size_t)4 * red_words + (size_t)4 * E) * sizeof(uint64_t) + ((size_t)E + 1) * sizeof(int32_t);
#define MOE_SELW(KPL)                                                                                              \
  hipLaunchKernelGGL((router_screen_select_wg_kernel<KPL, 4, 3>), dim3(T), dim3(256), lds, st, (const bf16_t*)x,     \
                     (const bf16_t*)w, bias, approx, absum, S, tok_off, T, d, E, scale, ids, wts, red_words)
    if (E <= 64) MOE_SELW(1);
    else if (E <= 128) MOE_SELW(2);
    else if (E <= 256) MOE_SELW(4);
    else if (E <= 512) MOE_SELW(8);
    else MOE_SELW(16);
#undef MOE_SELW
    return hipGetLastError();
  }
  dim3 grid((T + 3) / 4);
  const int red_words = max(SEL_GRP * 64, k_max + 1);
  const int words = red_words + (E + 1) / 2 + E;
  const size_t lds = (size_t)4 * words * sizeof(uint64_t);
#define MOE_SEL(KPL, XC)                                                                                          \
  launch_select<KPL, XC>(grid, lds, st, (const bf16_t*)x, (const bf16_t*)w, bias, approx, absum, S, tok_off, T, d, E, \
                         scale, ids, wts, red_words, words)
  if (E <= 64) MOE_SEL(1, 4);
  else if (E <= 128) MOE_SEL(2, 4);
  else if (E <= 256) MOE_SEL(4, 4);
  else if (E <= 512) MOE_SEL(8, 4);
  else MOE_SEL(16, 4);
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
