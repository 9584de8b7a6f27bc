// Training-free proxy gating of a split layer (MoE-Prism, arXiv 2510.19366,
// §III-B2, Training-Free Proxy Gating).
//
// Each whole expert e was cut into N sub-experts (index N*e + n).  The
// original router picks m whole experts per token; every sub-expert n of the
// j-th picked expert gets a proxy score, the mean |SiLU(g_c) u_c| over its r
// gate neurons c; the kappa_j best sub-experts run, each with the whole
// expert's routing weight.
//
// The proxy activations are a SwiGLU over a small gathered weight set: for
// whole expert e, rows n*r + i of wp_gate / wp_up are gate neuron i of
// sub-expert N*e + n, zero rows pad the set to Ip (N*r rounded up to the FFN
// kernels' dimension quantum).  proxy_pack_kernel gathers them once; the
// grouped FFN's gate/up kernel then produces every routed token's activations
// (hp, row stride Ip), and the kernels here turn them into routes:
//   proxy_offsets_kernel one workgroup: routes per token = its budget k_t =
//                        sum_j kappa_j, exclusive scan into tok_off;
//   proxy_select_kernel  one wave per token, lane j*N + n scores sub-expert n
//                        of pick j, ranks within its N lanes by shuffles and
//                        writes the chosen ones in (pick, score) order.
#include "common.h"
#include "launch.h"

namespace moe {

// ---- gather of the gate-neuron rows: one wave per packed row, 16 B per lane ----
// Packed row q of whole expert e (q < Ip): neuron i = q % r of sub-expert
// N*e + q / r while q < N*r, a zero row after that.  Source and packed
// matrices share the weight layout (`blocked`: w_offset in common.h).
template <typename T>
__global__ __launch_bounds__(256) void proxy_pack_kernel(const int32_t* __restrict__ gate_idx, const T* __restrict__ wg,
                                                         const T* __restrict__ wu, int E_base, int I_sub, int d, int N,
                                                         int r, int Ip, T* __restrict__ pg, T* __restrict__ pu,
                                                         int blocked) {
  constexpr int LE = 16 / sizeof(T);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= E_base * Ip) return;
  const int e = row / Ip, q = row - e * Ip;
  bool ok = q < N * r;
  size_t src = 0;
  int c = 0;
  if (ok) {
    const int sub = N * e + q / r;
    c = gate_idx[(size_t)sub * r + q % r];
    ok = c >= 0 && c < I_sub;
    if (!ok) c = 0;
    src = (size_t)sub * I_sub * d;
  }
  T* dg = pg + (size_t)e * Ip * d;
  T* du = pu + (size_t)e * Ip * d;
  for (int o = lane * LE; o < d; o += 64 * LE) {
    const size_t so = src + w_offset<T>(c, o, d, blocked), dof = w_offset<T>(q, o, d, blocked);
    const uint4 vg = ok ? *reinterpret_cast<const uint4*>(wg + so) : zero_u4();
    const uint4 vu = ok ? *reinterpret_cast<const uint4*>(wu + so) : zero_u4();
    *reinterpret_cast<uint4*>(dg + dof) = vg;
    *reinterpret_cast<uint4*>(du + dof) = vu;
  }
}

// A budget runs when 0 <= kt <= k_max and its kappa row is a valid split of
// it (every entry in [0, N], sum kt); otherwise the token runs nothing and the
// status is flagged.  A valid row keeps every token within k_max routes.
__device__ __forceinline__ bool budget_ok(const int32_t* __restrict__ kappa, int m, int N, int k_max, int kt) {
  if (kt < 0 || kt > k_max) return false;
  int sum = 0;
  for (int j = 0; j < m; ++j) {
    const int v = kappa[(size_t)kt * m + j];
    if (v < 0 || v > N) return false;
    sum += v;
  }
  return sum == kt;
}

// ---- routes per token and their offsets (one workgroup of 1024 threads) ----
// The budget check is done once per budget into LDS (runs[kt] = kt or -1), so
// that each token costs one LDS read.
__global__ __launch_bounds__(1024) void proxy_offsets_kernel(const int32_t* __restrict__ k,
                                                             const int32_t* __restrict__ kappa, int T, int k_max,
                                                             int m, int N, int32_t* __restrict__ tok_off,
                                                             int32_t* __restrict__ status) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t runs[65];
  __shared__ int32_t bad_any;
  const int tid = threadIdx.x;
  if (tid <= k_max) runs[tid] = budget_ok(kappa, m, N, k_max, tid) ? tid : -1;
  if (tid == 0) bad_any = 0;
  __syncthreads();
  auto routes = [&](int kt) { return (kt < 0 || kt > k_max) ? -1 : runs[kt]; };
  const int per = (T + 1023) / 1024;
  const int beg = min(tid * per, T), end = min(beg + per, T);
  int s = 0, bad = 0;
  for (int i = beg; i < end; ++i) {
    const int c = routes(k[i]);
    bad |= c < 0;
    s += max(c, 0);
  }
  if (bad) atomicOr(&bad_any, 1);
  const int incl = block_scan_incl<1024>(s, wsum);
  int run = incl - s;
  for (int i = beg; i < end; ++i) {
    tok_off[i] = run;
    run += max(routes(k[i]), 0);
  }
  if (tid == 1023) tok_off[T] = incl;
  if (tid == 0 && status) status[0] = bad_any ? MOE_DEV_BAD_K_BIT : 0;
}

// ---- selection: one wave per token, lane j*N + n ----
template <typename T>
__global__ __launch_bounds__(256) void proxy_select_kernel(
    const int32_t* __restrict__ k, const int32_t* __restrict__ kappa, int Tn, int k_max, int m, int N, int r, int Ip,
    const int32_t* __restrict__ base_tok_off, const int32_t* __restrict__ base_ids, const float* __restrict__ base_w,
    const int32_t* __restrict__ base_inv, const T* __restrict__ hp, int E_base, const int32_t* __restrict__ tok_off,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int kt = k[t];
  if (!budget_ok(kappa, m, N, k_max, kt)) return;
  const int j = lane / N, n = lane - j * N;
  const bool live = j < m;
  int e = 0, kj = 0, before = 0;
  float s = 0.f, wj = 0.f;
  if (live) {
    const int a = base_tok_off[t] + j;
    e = base_ids[a];
    wj = base_w[a];
    kj = kappa[(size_t)kt * m + j];
    for (int q = 0; q < j; ++q) before += kappa[(size_t)kt * m + q];
    if (e >= 0 && e < E_base) {
      const T* row = hp + (size_t)base_inv[a] * Ip + n * r;
      for (int i = 0; i < r; ++i) s += fabsf(Elt<T>::to_f32(row[i]));
      s /= (float)r;
    } else {
      // a pick outside the whole experts runs nothing: its kappa_j slots,
      // already counted in the offsets, become holes (id -1, weight 0) that
      // the permutation and the combine skip
      if (n < kj) {
        const int pos = tok_off[t] + before + n;
        ids[pos] = -1;
        wts[pos] = 0.f;
      }
      kj = 0;
    }
  }
  // rank among the N sub-experts of the same pick: larger score, then lower n
  int rank = 0;
  for (int q = 0; q < N; ++q) {
    const float sq = __shfl(s, j * N + q, 64);
    rank += (sq > s) || (sq == s && q < n);
  }
  if (live && rank < kj) {
    const int pos = tok_off[t] + before + rank;
    ids[pos] = N * e + n;
    wts[pos] = wj;
  }
}

hipError_t launch_proxy_pack(int dtype, const int32_t* gate_idx, const void* wg, const void* wu, int E_base, int I_sub,
                             int d, int N, int r, int Ip, void* pg, void* pu, int blocked, hipStream_t st) {
  const int64_t rows = (int64_t)E_base * Ip;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(proxy_pack_kernel<bf16_t>, grid, dim3(256), 0, st, gate_idx, (const bf16_t*)wg,
                       (const bf16_t*)wu, E_base, I_sub, d, N, r, Ip, (bf16_t*)pg, (bf16_t*)pu, blocked);
  else
    hipLaunchKernelGGL(proxy_pack_kernel<float>, grid, dim3(256), 0, st, gate_idx, (const float*)wg, (const float*)wu,
                       E_base, I_sub, d, N, r, Ip, (float*)pg, (float*)pu, blocked);
  return hipGetLastError();
}

hipError_t launch_proxy_route(int dtype, const int32_t* k, const int32_t* kappa, int T, int k_max, int m, int N, int r,
                              int Ip, const int32_t* base_tok_off, const int32_t* base_ids, const float* base_w,
                              const int32_t* base_inv, const void* hp, int E_base, int32_t* tok_off, int32_t* ids,
                              float* wts, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(proxy_offsets_kernel, dim3(1), dim3(1024), 0, st, k, kappa, T, k_max, m, N, tok_off, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || T == 0) return err;
  const dim3 grid((T + 3) / 4);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(proxy_select_kernel<bf16_t>, grid, dim3(256), 0, st, k, kappa, T, k_max, m, N, r, Ip, base_tok_off,
                       base_ids, base_w, base_inv, (const bf16_t*)hp, E_base, tok_off, ids, wts);
  else
    hipLaunchKernelGGL(proxy_select_kernel<float>, grid, dim3(256), 0, st, k, kappa, T, k_max, m, N, r, Ip, base_tok_off,
                       base_ids, base_w, base_inv, (const float*)hp, E_base, tok_off, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
