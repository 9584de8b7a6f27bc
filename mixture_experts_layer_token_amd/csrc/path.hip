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
// Source-grouped reuse then needs no kernel of its own: the expansions run as
// the grouped FFN's gate/up over the source routes, the projections as its
// down projection over the paths grouped by target, reading their expansion
// rows through the row map.
#include "common.h"
#include "launch.h"
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
