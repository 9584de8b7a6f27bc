// Device code shared by the two router kernels: the token-offset scan and
// the per-token top-k_t selection with its routing weights (one wave64 per
// token).
//
// Selection order (MoE-Prism, arXiv 2510.19366, §III-B2: the selected experts
// are ordered by router probability): logit descending, ties to the lower
// expert index, -0.0 equal to +0.0.  Lane l holds the keys of experts
// l, l + 64, ..., l + 64 * (KPL - 1).  A key is the order-preserving uint32
// image of the float32 logit; 0 marks an expert that cannot be selected.
//
// Steps, none of which moves keys between lanes:
//  1. V = k-th largest key, by a 32-step radix search: each step counts the
//     keys >= a trial value with one ballot per slot.
//  2. Selected = keys > V, then keys == V in ascending expert index until k.
//  3. The selected (key, expert) pairs are listed in LDS; each one's output
//     position is the number of listed pairs that precede it in the order.
//  4. Weights: p_j = exp(l_j - l_0) (l_0 the best logit), summed in a fixed
//     order (per lane in rank order, then a fixed butterfly read from lane 0),
//     w_j = scale * p_j / sum  -- the softmax renormalised over the selection.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

// tok_off = exclusive prefix sum of the executed budgets, by one workgroup of
// NT threads (each a contiguous run of tokens).  A k_t outside [0, k_max]
// counts as 0 and raises MOE_DEV_BAD_K; the policy then maps each valid
// budget to the one executed (BATCH_MAX: the largest valid budget of the
// batch; ROUND_UP: the next multiple of the granule, at most k_max when k_max
// is a multiple of it).  `part` holds NT / 64 ints, `bad_any` one.
__device__ __forceinline__ int budget_valid(int v, int k_max) { return v >= 0 && v <= k_max; }
__device__ __forceinline__ int budget_exec(int v, int k_max, BudgetPolicy pol, int kb) {
  if (!budget_valid(v, k_max)) return 0;
  if (pol.policy == K_BATCH_MAX) return kb;
  if (pol.policy == K_ROUND_UP) return (v + pol.granule - 1) / pol.granule * pol.granule;
  return v;
}

// A thread's first KR budgets are loaded once, together, and kept in
// registers for the three passes (batches up to KR * NT tokens never re-read).
template <int NT>
__device__ void token_offsets_block(const int32_t* __restrict__ k, int T, int k_max, BudgetPolicy pol,
                                    int32_t* __restrict__ tok_off, int32_t* __restrict__ status, int32_t* part,
                                    int32_t* bad_any) {
  constexpr int KR = 32;
  const int tid = threadIdx.x;
  const int per = (T + NT - 1) / NT;
  const int beg = min(tid * per, T), end = min(beg + per, T);
  int kr[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) kr[j] = (beg + j < end) ? k[beg + j] : 0;
  int bad = 0, kmx = 0;
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    if (beg + j < end) {
      const bool ok = budget_valid(kr[j], k_max);
      bad |= !ok;
      kmx = max(kmx, ok ? kr[j] : 0);
    }
  }
  for (int i = beg + KR; i < end; ++i) {
    const int v = k[i];
    const bool ok = budget_valid(v, k_max);
    bad |= !ok;
    kmx = max(kmx, ok ? v : 0);
  }
  // batch maximum of the valid budgets (only BATCH_MAX uses it)
  const int kb = pol.policy == K_BATCH_MAX ? block_max<NT>(kmx, part) : 0;
  int s = 0;
#pragma unroll
  for (int j = 0; j < KR; ++j)
    if (beg + j < end) s += budget_exec(kr[j], k_max, pol, kb);
  for (int i = beg + KR; i < end; ++i) s += budget_exec(k[i], k_max, pol, kb);
  if (tid == 0) *bad_any = 0;
  __syncthreads();
  if (bad) atomicOr(bad_any, 1);
  const int incl = block_scan_incl<NT>(s, part);  // its barriers also publish bad_any
  int run = incl - s;
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    if (beg + j < end) {
      tok_off[beg + j] = run;
      run += budget_exec(kr[j], k_max, pol, kb);
    }
  }
  for (int i = beg + KR; i < end; ++i) {
    tok_off[i] = run;
    run += budget_exec(k[i], k_max, pol, kb);
  }
  if (tid == NT - 1) tok_off[T] = incl;
  if (tid == 0 && status) status[0] = *bad_any ? MOE_DEV_BAD_K_BIT : 0;
}


__device__ __forceinline__ uint32_t logit_key(float l) {
  if (l == 0.0f) l = 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Number of keys >= v over the wave (every lane gets the same count).
template <int KPL>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&key)[KPL], uint32_t v) {
  int c = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s) c += __popcll(__ballot(key[s] >= v));
  return c;
}

// k-th largest key (1 <= k <= number of keys > 0); wave-uniform result.
template <int KPL>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t (&key)[KPL], int k) {
  uint32_t prefix = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t trial = prefix | (1u << b);
    if (wave_count_ge<KPL>(key, trial) >= k) prefix = trial;
  }
  return prefix;
}

// Marks the k selected slots: keys above V, then keys equal to V in ascending
// expert index (slot-major, then lane).
template <int KPL>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[KPL], int k, bool (&sel)[KPL]) {
  const int lane = threadIdx.x & 63;
  const uint32_t V = wave_kth_largest<KPL>(key, k);
  int need = k;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    sel[s] = key[s] > V;
    need -= __popcll(__ballot(sel[s]));
  }
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const uint64_t eq = __ballot(key[s] == V && key[s] != 0u);
    const int n_eq = __popcll(eq);
    if (need > 0 && key[s] == V && key[s] != 0u && __popcll(eq & below) < need) sel[s] = true;
    need -= min(need, n_eq);
  }
}

// Selects the top k (1 <= k <= present keys), calls emit(j, slot) for the
// selected key of this lane's slot `slot` that lands at position j, and writes
// wts[j], for j = 0 .. k-1 in selection order.  `scratch` is this wave's LDS
// area of at least k + 1 uint64 slots.
template <int KPL, class Emit>
__device__ __forceinline__ void wave_topk_softmax_emit(const uint32_t (&key)[KPL], int k, float scale, Emit emit,
                                                       float* __restrict__ wts, uint64_t* scratch) {
  const int lane = threadIdx.x & 63;
  bool sel[KPL];
  wave_select<KPL>(key, k, sel);
  // list the selected pairs (key high, inverted expert low: larger = earlier)
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const uint64_t m = __ballot(sel[s]);
    if (sel[s]) {
      const uint32_t e = (uint32_t)(lane + 64 * s);
      scratch[base + __popcll(m & below)] = ((uint64_t)key[s] << 32) | (uint64_t)(0xffffffffu - e);
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ranks; the best pair publishes its logit
  int rank[KPL];
  float* const l0slot = reinterpret_cast<float*>(scratch + k);
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    rank[s] = -1;
    if (sel[s]) {
      const uint32_t e = (uint32_t)(lane + 64 * s);
      const uint64_t me = ((uint64_t)key[s] << 32) | (uint64_t)(0xffffffffu - e);
      int r = 0;
      for (int j = 0; j < k; ++j) r += scratch[j] > me;
      rank[s] = r;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int s = 0; s < KPL; ++s)
    if (rank[s] == 0) *l0slot = key_logit(key[s]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float l0 = *l0slot;
  // p by rank into LDS (reusing the list), ids out
  float* const ps = reinterpret_cast<float*>(scratch);
  float p[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    p[s] = 0.f;
    if (rank[s] >= 0) {
      p[s] = expf(key_logit(key[s]) - l0);
      emit(rank[s], s);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int s = 0; s < KPL; ++s)
    if (rank[s] >= 0) ps[rank[s]] = p[s];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // fixed-order sum: lane i adds ranks i, i + 64, ... in order; then a butterfly
  float part = 0.f;
  for (int j = lane; j < k; j += 64) part += ps[j];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  const float sum = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(part)));
  const float inv = scale / sum;
#pragma unroll
  for (int s = 0; s < KPL; ++s)
    if (rank[s] >= 0) wts[rank[s]] = p[s] * inv;
}

// The same, writing ids[j] = the selected expert (lane + 64 * slot).
template <int KPL>
__device__ __forceinline__ void wave_topk_softmax(const uint32_t (&key)[KPL], int k, float scale,
                                                  int32_t* __restrict__ ids, float* __restrict__ wts,
                                                  uint64_t* scratch) {
  const int lane = threadIdx.x & 63;
  wave_topk_softmax_emit<KPL>(key, k, scale, [&](int j, int s) { ids[j] = lane + 64 * s; }, wts, scratch);
}

}  // namespace moe
