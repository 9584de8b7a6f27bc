// Compositional path routing and source-grouped execution metadata (PCoMoE,
// arXiv 2609.01024).
//
// Expert e splits at its expansion/projection boundary into U_e (the gate/up
// SwiGLU half) and D_e (the down projection); a path (i, j) is D_j(U_i(h)),
// the diagonal (e, e) the vanilla expert.  A fixed list of active paths
// (source, target, compatibility bias) is the candidate set.
//
//   path_topk_kernel        one wave per token: router logits g (and target
//                           prior logits t) from the float64 partial sums of
//                           the router's slices, path scores
//                           s = fp32((g[src] + b) + lambda * t[tgt]) in
//                           float64, top-k_t and softmax weights (select.h);
//   path_src_count_kernel   one wave per token: the distinct sources of its
//                           paths by an LDS bitmap over the experts, their
//                           count, each path's rank among them;
//   path_scan_kernel        one workgroup: exclusive scan of the counts;
//   path_src_place_kernel   one wave per token: sources into place, each
//                           path's source route, the one-path-per-row offsets;
//   path_rows_kernel        elementwise: the expansion row each
//                           target-ordered path reads.
//
//   path_screen_kernel      (large bf16 batches) the same selection from the
//                           screened router's MFMA pass: bounds on every
//                           path score, exact logits only for the sources and
//                           targets of the paths that can still be selected.
//
// Source-grouped reuse then needs no kernel of its own: the expansions run as
// the grouped FFN's gate/up over the source routes, the projections as its
// down projection over the paths grouped by target, reading their expansion
// rows through the row map.
#include "common.h"
#include "launch.h"
#include "screen.h"
#include "select.h"

namespace moe {

// ---- path scores and per-token top-k_t (one wave per token) ----
template <int KPL>
__global__ __launch_bounds__(256) void path_topk_kernel(const double* __restrict__ part_g,
                                                        const double* __restrict__ part_t, int S,
                                                        const float* __restrict__ bias, const int32_t* __restrict__ psrc,
                                                        const int32_t* __restrict__ ptgt, const float* __restrict__ pb,
                                                        int P, float lam, const int32_t* __restrict__ tok_off, int T,
                                                        int E, float scale, int32_t* __restrict__ osrc,
                                                        int32_t* __restrict__ otgt, float* __restrict__ wts,
                                                        int scratch_slots, int words) {
  extern __shared__ uint64_t path_lds[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  uint64_t* const scratch = path_lds + (size_t)wv * words;
  float* const gl = reinterpret_cast<float*>(scratch + scratch_slots);
  float* const tl = gl + E;
  // logits: the slices added in ascending order, the bias, one rounding (the
  // router's own arithmetic, so a diagonal path scores its expert's logit)
  const size_t qs = (size_t)T * E;
  for (int e = lane; e < E; e += 64) {
    double a = 0.0;
    const double* pg = part_g + (size_t)t * E + e;
    for (int q = 0; q < S; ++q) a += pg[q * qs];
    if (bias) a += (double)bias[e];
    gl[e] = (float)a;
    if (part_t) {
      double b = 0.0;
      const double* pt = part_t + (size_t)t * E + e;
      for (int q = 0; q < S; ++q) b += pt[q * qs];
      tl[e] = (float)b;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t key[KPL];
  int si[KPL], sj[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int p = lane + 64 * s;
    key[s] = 0;
    si[s] = sj[s] = 0;
    if (p < P) {
      si[s] = psrc[p];
      sj[s] = ptgt[p];
      double v = (double)gl[si[s]] + (double)pb[p];
      if (part_t) v += (double)lam * (double)tl[sj[s]];
      key[s] = logit_key((float)v);
    }
  }
  if (kt == 0) return;
  wave_topk_softmax_emit<KPL>(
      key, kt, scale,
      [&](int j, int s) {
        osrc[base + j] = si[s];
        otgt[base + j] = sj[s];
      },
      wts + base, scratch);
}

// ---- screened path selection (bf16, E <= 256), one wave per token ----
// Each logit lies within r = n * 2^-22 * sum|x||w| + n * 2^-126 of its MFMA
// value, n the summation depth of the screening pass (screen_depth: the
// screened router's bound), widened by 2^-22 of its size for the rounding of
// the exact logit to float32; the float32 logits g, t are then inside
// [lo, hi] rounded outwards.  A path score is a monotone function of (g, t),
// evaluated exactly as for the exact score, so its bounds are the function at
// the interval ends.  L = the k_t-th largest lower bound (rounded down to
// float32); a path whose upper bound is below L minus four float32 ulps is
// beaten by k_t paths whose scores are at least L, strictly: it cannot be
// selected.  The others get exact logits (float64 sums, screen.h) for their
// source and target, exact scores, and the selection of select.h on those.
// Groups of 4 rows in the cross-lane sums keep a wave's LDS area at ~8 KB
// (E = 256), four waves per workgroup.
constexpr int PS_GRP = 4;

template <int KPL, int KE, int XC, bool XR>
__global__ __launch_bounds__(256) void path_screen_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const bf16_t* __restrict__ wt,
    const float* __restrict__ bias, const float* __restrict__ ag, const float* __restrict__ sg,
    const float* __restrict__ at, const float* __restrict__ stt, int S, const int32_t* __restrict__ psrc,
    const int32_t* __restrict__ ptgt, const float* __restrict__ pb, int P, float lam,
    const int32_t* __restrict__ tok_off, int T, int d, int E, float scale, int32_t* __restrict__ osrc,
    int32_t* __restrict__ otgt, float* __restrict__ wts, int red_words, int words) {
  extern __shared__ uint64_t ps_lds[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  const bool has_t = wt != nullptr;
  // per-wave LDS: [red_words: row shares, later the top-k scratch][2E int32:
  // work list][E floats each: g lo, g hi, t lo, t hi -- the lo arrays then
  // hold the exact logits of the needed experts][2 x 256-bit masks: sources,
  // targets needed]
  uint64_t* const area = ps_lds + (size_t)wv * words;
  double* const red = reinterpret_cast<double*>(area);
  int32_t* const clist = reinterpret_cast<int32_t*>(area + red_words);
  float* const glo = reinterpret_cast<float*>(area + red_words + E);
  float* const ghi = glo + E;
  float* const tlo = ghi + E;
  float* const thi = tlo + E;
  float* const gx = glo;
  float* const tx = tlo;
  uint32_t* const need = reinterpret_cast<uint32_t*>(thi + E);
  const double depth = screen_depth(d, S);
  const double rad_scale = depth * 0x1p-22, rad_floor = depth * 0x1p-126;
  const size_t sstride = (size_t)T * E;
  const int nm = has_t ? 2 : 1;
  // slice partials of the lane's experts, all (expert, matrix) pairs of a
  // slice requested together, slices added in ascending order
  float sa[2][KE], sq[2][KE];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < KE; ++s) sa[m][s] = sq[m][s] = 0.f;
  for (int z = 0; z < S; ++z) {
    float va[2][KE], vq[2][KE];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < KE; ++s) {
        const int e = lane + 64 * s;
        const bool on = e < E && m < nm;
        const size_t off = (size_t)z * sstride + (size_t)t * E + (on ? e : 0);
        va[m][s] = on ? (m ? at : ag)[off] : 0.f;
        vq[m][s] = on ? (m ? stt : sg)[off] : 0.f;
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < KE; ++s) {
        sa[m][s] += va[m][s];
        sq[m][s] += vq[m][s];
      }
  }
#pragma unroll
  for (int s = 0; s < KE; ++s) {
    const int e = lane + 64 * s;
    if (e < E) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m >= nm) continue;
        const double c = (double)sa[m][s] + ((m == 0 && bias) ? (double)bias[e] : 0.0);
        const double r = rad_scale * (double)sq[m][s] + fabs(c) * 0x1p-22 + rad_floor;
        (m ? tlo : glo)[e] = __double2float_rd(c - r);
        (m ? thi : ghi)[e] = __double2float_ru(c + r);
      }
    }
  }
  if (lane < 16) need[lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (kt == 0) return;
  // Path data are re-read from the (cached) table in each phase rather than
  // kept in registers: with up to 16 slots per lane, registers are what
  // limits the waves per SIMD here.
  auto score_bounds = [&](int p, double& lo, double& hi) {
    const int i = psrc[p], j = ptgt[p];
    const double b = (double)pb[p];
    lo = (double)glo[i] + b;
    hi = (double)ghi[i] + b;
    if (has_t) {
      const double tl = (double)tlo[j], th = (double)thi[j];
      lo += (double)lam * (lam >= 0.f ? tl : th);
      hi += (double)lam * (lam >= 0.f ? th : tl);
    }
  };
  // L: the k_t-th largest lower bound, rounded down to float32
  float L;
  {
    uint32_t lkey[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const int p = lane + 64 * s;
      lkey[s] = 0;
      if (p < P) {
        double lo, hi;
        score_bounds(p, lo, hi);
        lkey[s] = logit_key(__double2float_rd(lo));
      }
    }
    L = key_logit(wave_kth_largest<KPL>(lkey, kt));
  }
  const double cut = (double)L - (fabs((double)L) * 0x1p-21 + 0x1p-126);
  uint32_t cand = 0;  // bit s: slot s can still be selected
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int p = lane + 64 * s;
    if (p < P) {
      double lo, hi;
      score_bounds(p, lo, hi);
      if (hi >= cut) {
        cand |= 1u << s;
        const int i = psrc[p], j = ptgt[p];
        atomicOr(&need[i >> 5], 1u << (i & 31));
        if (has_t) atomicOr(&need[8 + (j >> 5)], 1u << (j & 31));
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // work list: the needed sources, then the needed targets, ascending
  int n = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int m = 0; m < nm; ++m) {
#pragma unroll
    for (int s = 0; s < KE; ++s) {
      const int e = lane + 64 * s;
      const bool on = e < E && ((need[8 * m + (e >> 5)] >> (e & 31)) & 1u);
      const uint64_t mask = __ballot(on);
      if (on) clist[n + __popcll(mask & below)] = e | (m << 16);
      n += __popcll(mask);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // exact logits of the needed experts, over their (no longer needed) lower bounds
  exact_dots<XC, XR, PS_GRP, 2, true>(
      x + (size_t)t * d, d, n,
      [&](int c) {
        const int v = clist[c];
        return ((v >> 16) ? wt : wr) + (size_t)(v & 0xffff) * d;
      },
      red,
      [&](int c, double v) {
        const int u = clist[c], e = u & 0xffff;
        if (u >> 16) tx[e] = (float)v;
        else gx[e] = (float)(v + (bias ? (double)bias[e] : 0.0));
      });
  // exact scores of the candidates (the arithmetic of path_topk_kernel)
  uint32_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    key[s] = 0;
    if ((cand >> s) & 1u) {
      const int p = lane + 64 * s;
      double v = (double)gx[psrc[p]] + (double)pb[p];
      if (has_t) v += (double)lam * (double)tx[ptgt[p]];
      key[s] = logit_key((float)v);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  wave_topk_softmax_emit<KPL>(
      key, kt, scale,
      [&](int j, int s) {
        const int p = lane + 64 * s;
        osrc[base + j] = psrc[p];
        otgt[base + j] = ptgt[p];
      },
      wts + base, area);
}

// ---- distinct sources per token: LDS bitmap over the experts ----
// A token's paths number k_t <= 64, one per lane.  Its distinct sources, in
// ascending order, go to tmp[tok_off[t] ...]; path a gets its source's rank in
// p2s[a]; cnt[t] = the number of distinct sources.
__global__ __launch_bounds__(256) void path_src_count_kernel(const int32_t* __restrict__ tok_off,
                                                             const int32_t* __restrict__ psrc, int T, int E,
                                                             int32_t* __restrict__ cnt, int32_t* __restrict__ tmp,
                                                             int32_t* __restrict__ p2s) {
  __shared__ uint32_t bits[4][32];
  __shared__ int32_t pre[4][32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  const int nw = (E + 31) >> 5;
  if (lane < 32) bits[wv][lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool mine = lane < kt;
  int v = 0;
  if (mine) {
    v = min(max(psrc[base + lane], 0), E - 1);  // in range when it comes from moe_path_route
    atomicOr(&bits[wv][v >> 5], 1u << (v & 31));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // exclusive prefix of the words' popcounts (lanes 0..31)
  const int c = (lane < nw) ? __popc(bits[wv][lane]) : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if ((lane & 31) >= off) incl += o;
  }
  if (lane < 32) pre[wv][lane] = incl - c;
  const int total = __shfl(incl, 31, 64);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (mine) {
    const int r = pre[wv][v >> 5] + __popc(bits[wv][v >> 5] & ((1u << (v & 31)) - 1u));
    tmp[base + r] = v;  // lanes sharing a source write the same value
    p2s[base + lane] = r;
  }
  if (lane == 0) cnt[t] = total;
}

// ---- exclusive scan of the per-token counts (one workgroup of 1024) ----
__global__ __launch_bounds__(1024) void path_scan_kernel(const int32_t* __restrict__ cnt, int T,
                                                         int32_t* __restrict__ off) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  const int per = (T + 1023) / 1024;
  const int beg = min(tid * per, T), end = min(beg + per, T);
  int s = 0;
  for (int i = beg; i < end; ++i) s += cnt[i];
  const int incl = block_scan_incl<1024>(s, wsum);
  int run = incl - s;
  for (int i = beg; i < end; ++i) {
    off[i] = run;
    run += cnt[i];
  }
  if (tid == 1023) off[T] = incl;
}

// ---- sources into place, source route of each path, one-path-per-row offsets ----
__global__ __launch_bounds__(256) void path_src_place_kernel(const int32_t* __restrict__ tok_off,
                                                             const int32_t* __restrict__ src_off,
                                                             const int32_t* __restrict__ tmp, int T,
                                                             int32_t* __restrict__ src_ids, int32_t* __restrict__ p2s,
                                                             int32_t* __restrict__ unit_off) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const int base = tok_off[t];
  const int kt = tok_off[t + 1] - base;
  const int s0 = src_off[t];
  const int ns = src_off[t + 1] - s0;
  if (lane < ns) src_ids[s0 + lane] = tmp[base + lane];
  if (lane < kt) {
    p2s[base + lane] += s0;
    unit_off[base + lane] = base + lane;
  }
}

// unit_off[a] = A for a in [A, cap]: the rows past the last path are empty.
__global__ __launch_bounds__(256) void path_unit_tail_kernel(const int32_t* __restrict__ tok_off, int T, int cap,
                                                             int32_t* __restrict__ unit_off) {
  const int A = tok_off[T];
  for (int a = blockIdx.x * 256 + threadIdx.x; a <= cap; a += gridDim.x * 256)
    if (a >= A) unit_off[a] = A;
}

// ---- expansion row of each target-ordered path ----
__global__ __launch_bounds__(256) void path_rows_kernel(const int32_t* __restrict__ tok_off, int T, int cap,
                                                        const int32_t* __restrict__ perm_path,
                                                        const int32_t* __restrict__ p2s,
                                                        const int32_t* __restrict__ src_inv,
                                                        int32_t* __restrict__ row_map) {
  const int A = tok_off[T];
  for (int q = blockIdx.x * 256 + threadIdx.x; q < cap; q += gridDim.x * 256)
    if (q < A) row_map[q] = src_inv[p2s[perm_path[q]]];
}

hipError_t launch_path_topk(const double* part_g, const double* part_t, int S, const float* bias,
                            const void* table, int P, float lam, const int32_t* tok_off, int T, int E, int k_max,
                            float scale, int32_t* osrc, int32_t* otgt, float* wts, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int32_t* psrc = static_cast<const int32_t*>(table);
  const int32_t* ptgt = psrc + P;
  const float* pb = reinterpret_cast<const float*>(ptgt + P);
  const int slots = k_max + 1;
  const int words = slots + E;  // top-k scratch, then E float logits and E float priors
  const size_t lds = (size_t)4 * words * sizeof(uint64_t);
  const dim3 grid((T + 3) / 4);
#define MOE_PATH(KPL)                                                                                              \
  hipLaunchKernelGGL(path_topk_kernel<KPL>, grid, dim3(256), lds, st, part_g, part_t, S, bias, psrc, ptgt, pb, P, \
                     lam, tok_off, T, E, scale, osrc, otgt, wts, slots, words)
  if (P <= 64) MOE_PATH(1);
  else if (P <= 128) MOE_PATH(2);
  else if (P <= 256) MOE_PATH(4);
  else if (P <= 512) MOE_PATH(8);
  else MOE_PATH(16);
#undef MOE_PATH
  return hipGetLastError();
}

template <int KPL>
static void launch_screen_kpl(dim3 grid, size_t lds, hipStream_t st, const bf16_t* x, const bf16_t* wr,
                              const bf16_t* wt, const float* bias, const float* ag, const float* sg, const float* at,
                              const float* stt, int S, const int32_t* psrc, const int32_t* ptgt, const float* pb,
                              int P, float lam, const int32_t* tok_off, int T, int d, int E, float scale,
                              int32_t* osrc, int32_t* otgt, float* wts, int red_words, int words) {
  if (d <= 2048)
    hipLaunchKernelGGL((path_screen_kernel<KPL, 4, 4, true>), grid, dim3(256), lds, st, x, wr, wt, bias, ag, sg, at,
                       stt, S, psrc, ptgt, pb, P, lam, tok_off, T, d, E, scale, osrc, otgt, wts, red_words, words);
  else
    hipLaunchKernelGGL((path_screen_kernel<KPL, 4, 4, false>), grid, dim3(256), lds, st, x, wr, wt, bias, ag, sg, at,
                       stt, S, psrc, ptgt, pb, P, lam, tok_off, T, d, E, scale, osrc, otgt, wts, red_words, words);
}

hipError_t launch_path_screen(const void* x, const void* w_router, const void* w_tgt, const float* bias,
                              const float* ag, const float* sg, const float* at, const float* stt, int S,
                              const void* table, int P, float lam, const int32_t* tok_off, int T, int d, int E,
                              int k_max, float scale, int32_t* osrc, int32_t* otgt, float* wts, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (E > 256) return hipErrorInvalidValue;
  const int32_t* psrc = static_cast<const int32_t*>(table);
  const int32_t* ptgt = psrc + P;
  const float* pb = reinterpret_cast<const float*>(ptgt + P);
  const int red_words = max(PS_GRP * 64, k_max + 1);
  const int words = red_words + 3 * E + 8;
  const size_t lds = (size_t)4 * words * sizeof(uint64_t);
  const dim3 grid((T + 3) / 4);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* wr = static_cast<const bf16_t*>(w_router);
  const bf16_t* wt = static_cast<const bf16_t*>(w_tgt);
#define MOE_PSCR(KPL)                                                                                             \
  launch_screen_kpl<KPL>(grid, lds, st, xb, wr, wt, bias, ag, sg, at, stt, S, psrc, ptgt, pb, P, lam, tok_off, T, d, \
                         E, scale, osrc, otgt, wts, red_words, words)
  if (P <= 64) MOE_PSCR(1);
  else if (P <= 128) MOE_PSCR(2);
  else if (P <= 256) MOE_PSCR(4);
  else if (P <= 512) MOE_PSCR(8);
  else if (P <= 768) MOE_PSCR(12);
  else MOE_PSCR(16);
#undef MOE_PSCR
  return hipGetLastError();
}

hipError_t launch_path_sources(const int32_t* tok_off, const int32_t* psrc, int T, int E, int k_max, int32_t* cnt,
                               int32_t* tmp, int32_t* src_off, int32_t* src_ids, int32_t* p2s, int32_t* unit_off,
                               hipStream_t st) {
  const int cap = T * k_max;
  const dim3 grid((T + 3) / 4);
  if (T > 0) {
    hipLaunchKernelGGL(path_src_count_kernel, grid, dim3(256), 0, st, tok_off, psrc, T, E, cnt, tmp, p2s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(path_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, T, src_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (T > 0) {
    hipLaunchKernelGGL(path_src_place_kernel, grid, dim3(256), 0, st, tok_off, src_off, tmp, T, src_ids, p2s,
                       unit_off);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(path_unit_tail_kernel, dim3(min(1024, cap / 256 + 1)), dim3(256), 0, st, tok_off, T, cap,
                     unit_off);
  return hipGetLastError();
}

hipError_t launch_path_rows(const int32_t* tok_off, int T, int k_max, const int32_t* perm_path, const int32_t* p2s,
                            const int32_t* src_inv, int32_t* row_map, hipStream_t st) {
  const int cap = T * k_max;
  if (cap == 0) return hipSuccess;
  hipLaunchKernelGGL(path_rows_kernel, dim3(min(1024, (cap + 255) / 256)), dim3(256), 0, st, tok_off, T, cap,
                     perm_path, p2s, src_inv, row_map);
  return hipGetLastError();
}

}  // namespace moe
