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
// v_mfma_f32_32x32x16_bf16, K split over S slices (partial sums per slice, added
// in slice order by pass 2).  Products of bf16 values are exact in fp32, so in
// any summation order of depth n the error is at most n * u * S with
// u = 2^-24 (2^-23 if the hardware truncates) and S <= s / (1 - n u).  A slice
// holds at most Lmax = ceil(d / 64 / S) * 64 products, each added once (in
// whatever order the MFMA adds them), and pass 2 adds the S slice values in
// fp32: n <= Lmax + S.  The radius used is r = n * 2^-22 * s + n * 2^-126,
// which covers both roundings with a factor of two to spare, and a product
// flushed to zero below the normal range at most 2^-126 each.  (The bound
// n <= d held before as well; with S slices it is about S times tighter, so
// fewer logits need the exact pass: on 4,096 tokens, d = 7168, S = 4, the
// depth falls from 7,168 to 1,796.)
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

typedef float f32x16_t __attribute__((ext_vector_type(16)));


// ---- pass 1: partial approximate logits and |x||w| sums of one K slice.
// A workgroup of 8 waves covers 64 tokens x 256 experts of one K slice.  K
// advances 64 at a time through an LDS ring of STG stages (token rows 64 x
// 128 B and router rows 256 x 128 B per stage, 40 KB) filled by global->LDS
// DMA in whole 128-byte lines; wave w multiplies experts [32w, 32w + 32)
// against the 64 tokens with v_mfma_f32_32x32x16_bf16 (value and |x||w|
// sums), its fragments read from rows XOR-swizzled as in the grouped GEMM
// (lds_off).  One more slice index (z = S) holds the token-offset scan (pass
// 2 needs it) in its first workgroup; its other workgroups exit at once.
// The kernel this replaced read the operands straight into registers, 64
// bytes of each of 16 rows per load instruction, a pattern that moves
// L2-resident data into a CU at about a third of the rate of whole lines:
// 4,096 tokens x 256 experts, d = 7168, 73 -> 48 us.  Of the 48, ~12 us
// store the 32 MB of partial sums, ~7 us are the scan workgroup waiting for
// a CU after the tiles (run inside the first tile workgroup it cost more),
// ~6 us launch and barriers.
constexpr int SCR_NW = 8, SCR_TOK = 64, SCR_EXP = 256;
constexpr int SCR_XB = SCR_TOK * 128, SCR_SB = SCR_XB + SCR_EXP * 128;  // bytes per stage: 8 KB + 32 KB

template <int STG>
__global__ __launch_bounds__(64 * SCR_NW) void router_screen_tile_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int d, int E, float* __restrict__ approx,
    float* __restrict__ absum, const int32_t* __restrict__ k, int k_max, BudgetPolicy pol,
    int32_t* __restrict__ tok_off, int32_t* __restrict__ status) {
  static_assert(STG >= 2 && STG * SCR_SB <= 160 * 1024, "LDS ring");
  __shared__ __attribute__((aligned(1024))) char lds[STG * SCR_SB];
  if (blockIdx.z == gridDim.z - 1) {
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      int32_t* part = reinterpret_cast<int32_t*>(lds);
      token_offsets_block<64 * SCR_NW>(k, T, k_max, pol, tok_off, status, part, part + SCR_NW);
    }
    return;
  }
  if (T == 0) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int S = gridDim.z - 1, z = blockIdx.z;
  const int t0 = blockIdx.x * SCR_TOK, e0 = blockIdx.y * SCR_EXP;
  const int chunks = d / 64;
  const int k_beg = (int)(((long long)z * chunks) / S) * 64;
  const int k_end = (int)(((long long)(z + 1) * chunks) / S) * 64;
  const int nk = (k_end - k_beg) / 64;

  // DMA sources (rows clamped in range; results of clamped rows are not
  // stored): x rows 8*wave .. +7, router rows 8*(j*8 + wave) .. +7
  const int rsub = lane >> 3;
  const bf16_t* xsrc;
  {
    const int r = 8 * wave + rsub;
    const int c = (lane & 7) ^ lds_swz(r);
    xsrc = x + (size_t)min(t0 + r, T - 1) * d + k_beg + c * 8;
  }
  const bf16_t* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (j * SCR_NW + wave) + rsub;
    const int c = (lane & 7) ^ lds_swz(r);
    wsrc[j] = w + (size_t)min(e0 + r, E - 1) * d + k_beg + c * 8;
  }
  auto issue = [&](int st) {
    char* sb = lds + (st % STG) * SCR_SB;
    const int ko = st * 64;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(xsrc + ko), (lds_ptr_t)(sb + wave * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wsrc[j] + ko), (lds_ptr_t)(sb + SCR_XB + (j * SCR_NW + wave) * 1024),
                                       16, 0, 0);
  };
  constexpr int PER = 5;  // DMA instructions per wave per stage

  f32x16_t acc[2], aab[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[i][e] = 0.f;
      aab[i][e] = 0.f;
    }
  const u32x4_t sign_off = {0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
  // Schedule of the grouped GEMM: the fragments of k16 step s+1 are read
  // during the MFMAs of step s; the barrier that hands over stage kt+1 sits
  // before the last step of stage kt, after which stage kt's buffer (its last
  // fragments are in registers) is refilled with stage kt + STG.
  u32x4_t fw[2], fx[2][2];
  auto load_frags = [&](int kt, int s, int slot) {
    const char* sb = lds + (kt % STG) * SCR_SB;
    fw[slot] = *reinterpret_cast<const u32x4_t*>(sb + SCR_XB + lds_off(32 * wave + l32, 2 * s + lh));
#pragma unroll
    for (int i = 0; i < 2; ++i) fx[slot][i] = *reinterpret_cast<const u32x4_t*>(sb + lds_off(32 * i + l32, 2 * s + lh));
  };
  auto mma = [&](int slot) {
    const u32x4_t aw = fw[slot] & sign_off;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fw[slot]),
                                                       __builtin_bit_cast(bf16x8_t, fx[slot][i]), acc[i], 0, 0, 0);
      aab[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                       __builtin_bit_cast(bf16x8_t, fx[slot][i] & sign_off), aab[i], 0,
                                                       0, 0);
    }
  };
  if (nk > 0) {
#pragma unroll
    for (int p = 0; p < STG; ++p)
      if (p < nk) issue(p);
    vm_wait_dyn<PER * (STG - 1)>(PER * min(STG - 1, nk - 1));  // stage 0 landed
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    load_frags(0, 0, 0);
  }
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) {
        load_frags(kt, s + 1, (s + 1) & 1);
      } else {
        // stage kt+1 landed (stages up to kt + STG - 1 may be in flight) and
        // this wave's reads of stage kt are complete; on the last stage the
        // reads below touch a buffer whose values are never used
        vm_wait_dyn<PER * (STG - 2)>(kt + 1 < nk ? PER * min(STG - 2, nk - 2 - kt) : 0);
        lgkm_wait0();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (kt + STG < nk) issue(kt + STG);
        load_frags(kt + 1, 0, 0);
      }
      mma(s & 1);
    }
  }
  // element e of acc[i] is D[n = 8*(e/4) + 4*lh + e%4][m = l32]: expert
  // e0 + 32*wave + n, token t0 + 32*i + m
  float* const ap = approx + (size_t)z * T * E;
  float* const sp = absum + (size_t)z * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 32 * i + l32;
    if (t >= T) continue;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int e = e0 + 32 * wave + 8 * e4 + 4 * lh;
      if ((E & 3) == 0 && e + 3 < E) {
        *reinterpret_cast<float4*>(ap + (size_t)t * E + e) =
            make_float4(acc[i][4 * e4], acc[i][4 * e4 + 1], acc[i][4 * e4 + 2], acc[i][4 * e4 + 3]);
        *reinterpret_cast<float4*>(sp + (size_t)t * E + e) =
            make_float4(aab[i][4 * e4], aab[i][4 * e4 + 1], aab[i][4 * e4 + 2], aab[i][4 * e4 + 3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < E) {
            ap[(size_t)t * E + e + r] = acc[i][4 * e4 + r];
            sp[(size_t)t * E + e + r] = aab[i][4 * e4 + r];
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
  const double depth = screen_depth(d, S);
  const double rad_scale = depth * 0x1p-22, rad_floor = depth * 0x1p-126;
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
      rad[s] = rad_scale * (double)m + rad_floor;
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

  // exact logits of the candidates (a resident row is kept as bf16 words, 3
  // candidates' rows in flight: 128 registers, 4 waves per SIMD; 8,192 tokens
  // x 256 experts, d = 2048: 161 -> 145 us for the whole route call)
  exact_dots<XC, XR, SEL_GRP, XR ? 3 : 2, true>(
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
    const double depth = screen_depth(d, S);
    const double rad_scale = depth * 0x1p-22, rad_floor = depth * 0x1p-126;
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
        rad[s] = rad_scale * (double)m + rad_floor;
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
// one, at least one 64-element stage per slice, and at most 2^22 partial
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
  if (d % 64 != 0) return hipErrorInvalidValue;  // d is a multiple of 128 for any valid descriptor
  const dim3 grid(max(1, (T + 63) / 64), (E + 255) / 256, S + 1);
  hipLaunchKernelGGL((router_screen_tile_kernel<3>), grid, dim3(64 * SCR_NW), 0, st, (const bf16_t*)x,
                     (const bf16_t*)w, T, d, E, approx, absum, k, k_max, pol, tok_off, status);
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
