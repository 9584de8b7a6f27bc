// Expert folding of the routing metadata (ExFold summary, arXiv 2608.24938:
// Unified Expert Folding; Phase-Specific Selection and Unified Folding;
// Phase-Specific Routing and Folding).
//
// The routes of a token are cut to a budget -- K routes per token, or only the
// experts of a batch-wide pool of D -- and every dropped route is folded into
// a kept target: the target of smallest projection loss L[source][target]
// receives the dropped weight times the scalar projector S[source][target].
// Only metadata changes, so the grouped FFN then runs the kept experts alone.
//
// Kernels:
//   fold_pool_kernel   (pool mode) one workgroup: per-expert aggregate
//                      H[e] * sum of routed weights (float64, in the rows'
//                      token order), the pool by rank counting, and the pool's
//                      member list in ascending expert order;
//   fold_routes_kernel one wave per token, one route per lane: keep / target /
//                      merge decisions by shuffles, folded routes written at
//                      the token's original offset, their count to cnt[t];
//   fold_scan_kernel   one workgroup: tok_off_out = exclusive scan of cnt (for
//                      at most 1024 tokens it also moves the routes);
//   fold_copy_kernel   one wave per token: routes to their final offsets.
// Every decision is a comparison of float32 values (scores are float32
// products, losses as stored) or of the float64 aggregates, taken in a fixed
// order; weights are added in route order.  Bit-reproducible.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int FOLD_MAX_K = 64;  // routes per token (one lane each)

// ---- pool selection (one workgroup of 1024 threads, E <= 1024) ----
// The routed weights are gathered into LDS in row (expert, token) order,
// FOLD_CHUNK rows at a time, by all threads; each expert's thread then adds
// its rows in order from LDS.
constexpr int FOLD_CHUNK = 16384;

__global__ __launch_bounds__(1024) void fold_pool_kernel(const float* __restrict__ H,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ expert_off,
                                                         const int32_t* __restrict__ perm_src, int E, int D,
                                                         int32_t* __restrict__ pool, int32_t* __restrict__ members,
                                                         int32_t* __restrict__ n_members,
                                                         int32_t* __restrict__ pool_out) {
  __shared__ float wl[FOLD_CHUNK];
  __shared__ double agg[1024];
  __shared__ int32_t act[1024];
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  const int A = expert_off[E];
  int p0 = 0, p1 = 0;
  if (e < E) {
    p0 = expert_off[e];
    p1 = expert_off[e + 1];
  }
  double s = 0.0;
  for (int c0 = 0; c0 < A; c0 += FOLD_CHUNK) {
    const int n = min(FOLD_CHUNK, A - c0);
    for (int i = e; i < n; i += 1024) wl[i] = w[perm_src[c0 + i]];
    __syncthreads();
    const int b = max(p0, c0), t = min(p1, c0 + n);
    for (int p = b; p < t; ++p) s += (double)wl[p - c0];
    __syncthreads();
  }
  const double a = e < E ? s * (double)H[e] : 0.0;
  const int on = p1 > p0;
  agg[e] = a;
  act[e] = on;
  __syncthreads();
  // rank among the activated experts: larger aggregate first, then lower index
  int r = 0;
  if (on) {
    for (int j = 0; j < E; ++j) r += act[j] && (agg[j] > a || (agg[j] == a && j < e));
  }
  const int in = on && r < D;
  if (e < E) {
    pool[e] = in;
    if (pool_out) pool_out[e] = in;
  }
  const int incl = block_scan_incl<1024>(in, wsum);
  if (in) members[incl - 1] = e;
  if (e == 1023) n_members[0] = incl;
}

// ---- per-token folding: one wave per token, lane j holds route j ----
template <int MODE>
__global__ __launch_bounds__(256) void fold_routes_kernel(
    const float* __restrict__ S, const float* __restrict__ L, const float* __restrict__ H,
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ ids, const float* __restrict__ w, int T, int E,
    int K, const int32_t* __restrict__ pool, const int32_t* __restrict__ members,
    const int32_t* __restrict__ n_members, int32_t* __restrict__ ids_tmp, float* __restrict__ w_tmp,
    int32_t* __restrict__ cnt) {
  __shared__ int32_t kept_e[4][FOLD_MAX_K];
  __shared__ int32_t mem_l[MODE == 1 ? 1024 : 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  int nm = 0;
  if (MODE == 1) {
    nm = n_members[0];
    for (int i = threadIdx.x; i < nm; i += 256) mem_l[i] = members[i];
    __syncthreads();
  }
  if (t >= T) return;
  const int a0 = tok_off[t];
  const int kt = min(tok_off[t + 1] - a0, FOLD_MAX_K);
  const bool live = lane < kt;
  int e = live ? ids[a0 + lane] : -1;
  const bool valid = live && e >= 0 && e < E;
  if (!valid) e = -1;
  const float wj = valid ? w[a0 + lane] : 0.f;
  const uint64_t below = (1ull << lane) - 1ull;

  int tgt = -1;      // expert this route ends on (-1: dropped without target)
  float c = 0.f;     // its contribution there
  bool emit;         // this lane writes an output route
  if (MODE == 0) {
    // keep the K largest scores (ties: earlier route); invalid routes last
    const float score = valid ? wj * H[e] : -1.f;
    int rank = 0;
    for (int i = 0; i < kt; ++i) {
      const float si = __shfl(score, i, 64);
      rank += (si > score) || (si == score && i < lane);
    }
    const bool kept = valid && (kt <= K || rank < K);
    const uint64_t km = __ballot(kept);
    const int nk = __popcll(km);
    if (kept) kept_e[wv][__popcll(km & below)] = e;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (kept) {
      tgt = e;
      c = wj;
    } else if (valid && nk > 0) {
      // the kept route of smallest L[e][.] (ties: earlier kept route)
      const float* Lr = L + (size_t)e * E;
      int best = 0;
      float bl = Lr[kept_e[wv][0]];
      for (int m = 1; m < nk; ++m) {
        const float l = Lr[kept_e[wv][m]];
        if (l < bl) {
          bl = l;
          best = m;
        }
      }
      tgt = kept_e[wv][best];
      c = wj * S[(size_t)e * E + tgt];
    }
    emit = kept;
  } else {
    const bool in_pool = valid && pool[e];
    if (in_pool) {
      tgt = e;
      c = wj;
    } else if (valid) {
      if (nm > 0) {
        const float* Lr = L + (size_t)e * E;
        int best = mem_l[0];
        float bl = Lr[best];
#pragma unroll 8
        for (int m = 1; m < nm; ++m) {
          const int p = mem_l[m];
          const float l = Lr[p];
          if (l < bl) {
            bl = l;
            best = p;
          }
        }
        tgt = best;
        c = wj * S[(size_t)e * E + tgt];
      }
    }
    // the first route landing on an expert carries the merged route
    bool first = tgt >= 0;
    for (int i = 0; i < kt; ++i) {
      const int ti = __shfl(tgt, i, 64);
      first = first && !(i < lane && ti == tgt);
    }
    emit = first;
  }
  // weight of an emitted route: its own contribution plus the routes folded
  // onto it, added in route order
  float acc = 0.f;
  for (int i = 0; i < kt; ++i) {
    const int ti = __shfl(tgt, i, 64);
    const float ci = __shfl(c, i, 64);
    if (emit && ti == tgt) acc += ci;
  }
  const uint64_t em = __ballot(emit);
  if (emit) {
    const int pos = __popcll(em & below);
    ids_tmp[a0 + pos] = tgt;
    w_tmp[a0 + pos] = acc;
  }
  if (lane == 0) cnt[t] = __popcll(em);
}

// ---- tok_off_out = exclusive scan of cnt (one workgroup; a thread owns a
// contiguous run of tokens).  COPY: the same threads also move their tokens'
// routes to the final offsets (small batches); else fold_copy_kernel does. ----
template <bool COPY>
__global__ __launch_bounds__(1024) void fold_scan_kernel(const int32_t* __restrict__ cnt,
                                                         const int32_t* __restrict__ tok_off, int T,
                                                         const int32_t* __restrict__ ids_tmp,
                                                         const float* __restrict__ w_tmp,
                                                         int32_t* __restrict__ tok_off_out,
                                                         int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  const int per = (T + 1023) / 1024;
  const int beg = min(tid * per, T), end = min(beg + per, T);
  int s = 0;
  for (int i = beg; i < end; ++i) s += cnt[i];
  const int incl = block_scan_incl<1024>(s, wsum);
  int run = incl - s;
  for (int i = beg; i < end; ++i) {
    const int n = cnt[i];
    tok_off_out[i] = run;
    if (COPY) {
      const int a0 = tok_off[i];
      for (int j = 0; j < n; ++j) {
        ids_out[run + j] = ids_tmp[a0 + j];
        w_out[run + j] = w_tmp[a0 + j];
      }
    }
    run += n;
  }
  if (tid == 1023) tok_off_out[T] = incl;
}

// ---- routes to their final offsets: one wave per token ----
__global__ __launch_bounds__(256) void fold_copy_kernel(const int32_t* __restrict__ tok_off,
                                                        const int32_t* __restrict__ tok_off_out, int T,
                                                        const int32_t* __restrict__ ids_tmp,
                                                        const float* __restrict__ w_tmp,
                                                        int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int a0 = tok_off[t], b0 = tok_off_out[t], n = tok_off_out[t + 1] - b0;
  for (int j = lane; j < n; j += 64) {
    ids_out[b0 + j] = ids_tmp[a0 + j];
    w_out[b0 + j] = w_tmp[a0 + j];
  }
}

hipError_t launch_fold(int mode, int budget, const float* S, const float* L, const float* H, const int32_t* tok_off,
                       const int32_t* ids, const float* w, const int32_t* expert_off, const int32_t* perm_src, int T,
                       int E, int32_t* tok_off_out, int32_t* ids_out, float* w_out, int32_t* pool_out,
                       const FoldScratch& ws, hipStream_t st) {
  if (mode == 1) {
    hipLaunchKernelGGL(fold_pool_kernel, dim3(1), dim3(1024), 0, st, H, w, expert_off, perm_src, E, budget, ws.pool,
                       ws.members, ws.n_members, pool_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (T > 0) {
    const dim3 grid((T + 3) / 4);
    if (mode == 0)
      hipLaunchKernelGGL(fold_routes_kernel<0>, grid, dim3(256), 0, st, S, L, H, tok_off, ids, w, T, E, budget,
                         ws.pool, ws.members, ws.n_members, ws.ids, ws.w, ws.cnt);
    else
      hipLaunchKernelGGL(fold_routes_kernel<1>, grid, dim3(256), 0, st, S, L, H, tok_off, ids, w, T, E, budget,
                         ws.pool, ws.members, ws.n_members, ws.ids, ws.w, ws.cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (T <= 1024) {  // one token per thread at most: copy in the scan
    hipLaunchKernelGGL(fold_scan_kernel<true>, dim3(1), dim3(1024), 0, st, ws.cnt, tok_off, T, ws.ids, ws.w,
                       tok_off_out, ids_out, w_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fold_scan_kernel<false>, dim3(1), dim3(1024), 0, st, ws.cnt, tok_off, T, ws.ids, ws.w,
                     tok_off_out, ids_out, w_out);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fold_copy_kernel, dim3((T + 3) / 4), dim3(256), 0, st, tok_off, tok_off_out, T, ws.ids, ws.w,
                     ids_out, w_out);
  return hipGetLastError();
}

}  // namespace moe
