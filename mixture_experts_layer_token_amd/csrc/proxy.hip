// Training-free proxy gating of a split layer (MoE-Prism, arXiv 2510.19366,
// §III-B2, Training-Free Proxy Gating).
//
// Each whole expert e was cut into N sub-experts (index N*e + n).  The
// original router picks m whole experts per token; every sub-expert n of the
// j-th picked expert gets a proxy score, the mean |SiLU(g_c) u_c| over its r
// gate neurons c; the kappa_j best sub-experts run, each with the whole
// expert's routing weight.
//
// Scores are taken on an exact basis, as the router's logits are: each gate
// neuron's pre-activations g = x . w_gate[c] and u = x . w_up[c] are exact
// products summed in float64 and rounded once to float32; the activation
// |SiLU(g) u| and the mean over the r neurons (in neuron order) are float64,
// and the picks are decided on those float64 scores (ties: lower n), so the
// choice is a function of the inputs alone, not of a kernel's summation
// order.
//
// For whole expert e, rows n*r + i of wp_gate / wp_up are gate neuron i of
// sub-expert N*e + n (proxy_pack_kernel gathers them once per layer; zero rows
// pad the set to Ip, N*r rounded up to the FFN kernels' dimension quantum).
//   proxy_offsets_kernel one workgroup: routes per token = its budget k_t =
//                        sum_j kappa_j, exclusive scan into tok_off;
//   proxy_holes_kernel   the slots of a pick outside the whole experts;
//   proxy_block_kernel   one workgroup per block of up to 64 rows of the
//                        whole-expert routes permuted by expert (all rows of
//                        one expert e): the exact dot products of the rows'
//                        tokens with e's gate-neuron rows, from tiles staged
//                        in LDS, then per row the scores of e's sub-experts
//                        and the kappa_j best of them, written in score order.
#include <algorithm>

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

// ---- holes: a pick outside the whole experts (one thread per (token, pick)) ----
// Such a pick has no row in the permutation and runs nothing: its kappa_j
// slots, counted in the offsets, become holes (id -1, weight 0) that the
// permutation and the combine skip.
__global__ __launch_bounds__(256) void proxy_holes_kernel(const int32_t* __restrict__ k,
                                                          const int32_t* __restrict__ kappa, int T, int k_max, int m,
                                                          int N, const int32_t* __restrict__ base_tok_off,
                                                          const int32_t* __restrict__ base_ids, int E_base,
                                                          const int32_t* __restrict__ tok_off,
                                                          int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)T * m) return;
  const int t = (int)(q / m), j = (int)(q - (int64_t)t * m);
  const int e = base_ids[base_tok_off[t] + j];
  if (e >= 0 && e < E_base) return;
  const int kt = k[t];
  if (!budget_ok(kappa, m, N, k_max, kt)) return;
  int pos = tok_off[t];
  for (int p = 0; p < j; ++p) pos += kappa[(size_t)kt * m + p];
  for (int p = 0; p < kappa[(size_t)kt * m + j]; ++p) {
    ids[pos + p] = -1;
    wts[pos + p] = 0.f;
  }
}

// ---- scoring and selection: one workgroup per row block of the base permutation ----
constexpr int PX_ROWS = 64;    // rows (routed (token, pick) pairs of one expert) per block
constexpr int PX_NG = 16;      // gate neurons per pass: 16 gate rows and 16 up rows
constexpr int PX_KC = 64;      // elements of K per LDS tile
constexpr int PX_XP = PX_KC + 2;  // x tile pitch in elements: an odd number of dwords per bf16 row
constexpr int PX_WP = PX_KC + 2;  // weight tile pitch in doubles

// Block b of the base permutation: the blocks of expert e (ceil(count_e / 64)
// of them) follow those of the lower experts.  Returns false past the last.
__device__ __forceinline__ bool proxy_block_of(const int32_t* __restrict__ eoff, int E_base, int b, int& e, int& r0,
                                               int& rows, int32_t* part, int32_t* found) {
  const int tid = threadIdx.x;
  if (tid == 0) found[0] = -1;
  int nb = 0;
  const int per = (E_base + 255) / 256, beg = min(tid * per, E_base), end = min(beg + per, E_base);
  for (int g = beg; g < end; ++g) nb += (eoff[g + 1] - eoff[g] + PX_ROWS - 1) / PX_ROWS;
  int run = block_scan_incl<256>(nb, part) - nb;
  for (int g = beg; g < end; ++g) {
    const int c = (eoff[g + 1] - eoff[g] + PX_ROWS - 1) / PX_ROWS;
    if (b >= run && b < run + c) {
      found[0] = g;
      found[1] = eoff[g] + (b - run) * PX_ROWS;
      found[2] = min(PX_ROWS, eoff[g + 1] - found[1]);
    }
    run += c;
  }
  __syncthreads();
  e = found[0];
  r0 = found[1];
  rows = found[2];
  return e >= 0;
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__global__ __launch_bounds__(256) void proxy_block_kernel(
    const int32_t* __restrict__ k, const int32_t* __restrict__ kappa, int k_max, int m, int N, int r, int Ip,
    const int32_t* __restrict__ base_tok_off, const float* __restrict__ base_w, const int32_t* __restrict__ base_eoff,
    const int32_t* __restrict__ base_ptok, const int32_t* __restrict__ base_psrc, const T* __restrict__ x,
    const T* __restrict__ wpg, const T* __restrict__ wpu, int E_base, int d, int blocked,
    const int32_t* __restrict__ tok_off, int32_t* __restrict__ ids, float* __restrict__ wts) {
  constexpr int LE = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T xs[PX_ROWS * PX_XP];
  __shared__ __attribute__((aligned(16))) double wsd[2 * PX_NG * PX_WP];  // the pass's weights, widened once
  __shared__ double act[PX_ROWS][PX_NG];
  __shared__ int32_t tok[PX_ROWS];
  __shared__ int32_t part[4], found[3];
  extern __shared__ double score[];  // [PX_ROWS][N], dynamic: N doubles a row
  int e, r0, rows;
  if (!proxy_block_of(base_eoff, E_base, blockIdx.x, e, r0, rows, part, found)) return;  // uniform
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < PX_ROWS) tok[tid] = base_ptok[r0 + (tid < rows ? tid : 0)];
  for (int q = tid; q < PX_ROWS * N; q += 256) score[q] = 0.0;
  __syncthreads();
  const size_t es = (size_t)e * Ip * d;
  const int NR = N * r;
  // Wave w: rows 16w .. 16w + 15 against the pass's 16 gate and 16 up rows,
  // two 16 x 16 float64 tiles, K in steps of 4 (v_mfma_f64_16x16x4f64: lane l
  // supplies row l % 16 at k = l / 16 of each operand; its output v is row
  // l / 16 + 4 v, column l % 16 -- unlike the float32 16 x 16 shapes, whose
  // output v of lane l is row 4 (l / 16) + v).
  const int ar = 16 * wave + (lane & 15), ak = lane >> 4;
  for (int c0 = 0; c0 < NR; c0 += PX_NG) {
    f64x4_t g = {0.0, 0.0, 0.0, 0.0}, u = {0.0, 0.0, 0.0, 0.0};
    // Each thread stages XQ 16-byte pieces of the x tile and WQ of the weight
    // tile per chunk; the pieces of chunk k0 + PX_KC are loaded into registers
    // before the products of chunk k0, so that their latency overlaps them.
    constexpr int XQ = PX_ROWS * (PX_KC / LE) / 256, WQ = 2 * PX_NG * (PX_KC / LE) / 256;
    static_assert(XQ * 256 == PX_ROWS * (PX_KC / LE) && WQ * 256 == 2 * PX_NG * (PX_KC / LE), "whole pieces");
    uint4 xv[XQ], wv[WQ];
    auto fetch = [&](int k0) {
#pragma unroll
      for (int p = 0; p < XQ; ++p) {
        const int q = tid + 256 * p, row = q / (PX_KC / LE), ch = q % (PX_KC / LE);
        xv[p] = *reinterpret_cast<const uint4*>(x + (size_t)tok[row] * d + k0 + ch * LE);
      }
#pragma unroll
      for (int p = 0; p < WQ; ++p) {
        const int q = tid + 256 * p, row = q / (PX_KC / LE), ch = q % (PX_KC / LE);
        const int c = c0 + (row % PX_NG);
        const T* src = (row < PX_NG ? wpg : wpu) + es;
        wv[p] = c < NR ? *reinterpret_cast<const uint4*>(src + w_offset<T>(c, k0 + ch * LE, d, blocked)) : zero_u4();
      }
    };
    fetch(0);
    for (int k0 = 0; k0 < d; k0 += PX_KC) {
      // the x rows (64 x 64 elements) and the pass's gate / up rows (32 x 64, widened to float64)
#pragma unroll
      for (int p = 0; p < XQ; ++p) {
        const int q = tid + 256 * p, row = q / (PX_KC / LE), ch = q % (PX_KC / LE);
        uint32_t* dst = reinterpret_cast<uint32_t*>(xs + row * PX_XP + ch * LE);
        dst[0] = xv[p].x;
        dst[1] = xv[p].y;
        dst[2] = xv[p].z;
        dst[3] = xv[p].w;
      }
#pragma unroll
      for (int p = 0; p < WQ; ++p) {
        const int q = tid + 256 * p, row = q / (PX_KC / LE), ch = q % (PX_KC / LE);
        const T* ve = reinterpret_cast<const T*>(&wv[p]);
#pragma unroll
        for (int q2 = 0; q2 < LE; ++q2) wsd[row * PX_WP + ch * LE + q2] = (double)Elt<T>::to_f32(ve[q2]);
      }
      __syncthreads();
      if (k0 + PX_KC < d) fetch(k0 + PX_KC);
#pragma unroll 4
      for (int kk = 0; kk < PX_KC; kk += 4) {
        // products of two float32 (or bfloat16) values are exact in float64
        const double a = (double)Elt<T>::to_f32(xs[ar * PX_XP + kk + ak]);
        const double bg = wsd[(lane & 15) * PX_WP + kk + ak];
        const double bu = wsd[(PX_NG + (lane & 15)) * PX_WP + kk + ak];
        g = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bg, g, 0, 0, 0);
        u = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bu, u, 0, 0, 0);
      }
      __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double g32 = (double)(float)g[v], u32 = (double)(float)u[v];  // one rounding to float32 each
      act[16 * wave + (lane >> 4) + 4 * v][lane & 15] = fabs(g32 / (1.0 + exp(-g32)) * u32);
    }
    __syncthreads();
    // each row adds its activations to its sub-experts' sums in neuron order
    if (tid < PX_ROWS)
      for (int q = 0; q < PX_NG && c0 + q < NR; ++q) score[tid * N + (c0 + q) / r] += act[tid][q];
    __syncthreads();
  }
  if (tid >= rows) return;
  // row tid: the (token, pick j) pair it routes, its budget's kappa_j
  const int t = tok[tid], a = base_psrc[r0 + tid];
  const int j = a - base_tok_off[t], kt = k[t];
  if (!budget_ok(kappa, m, N, k_max, kt)) return;
  const int kj = kappa[(size_t)kt * m + j];
  int before = 0;
  for (int q = 0; q < j; ++q) before += kappa[(size_t)kt * m + q];
  const int pos0 = tok_off[t] + before;
  const float wj = base_w[a];
  // the kappa_j best sub-experts by score (larger, then lower n), in score order
  double* const sc = score + tid * N;
  for (int n = 0; n < N; ++n) sc[n] /= (double)r;
  for (int n = 0; n < N; ++n) {
    const double sn = sc[n];
    int rank = 0;
    for (int q = 0; q < N; ++q) rank += (sc[q] > sn) || (sc[q] == sn && q < n);
    if (rank < kj) {
      ids[pos0 + rank] = N * e + n;
      wts[pos0 + rank] = wj;
    }
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
                              const int32_t* base_eoff, const int32_t* base_ptok, const int32_t* base_psrc,
                              const void* x, const void* wpg, const void* wpu, int E_base, int d, int blocked,
                              int32_t* tok_off, int32_t* ids, float* wts, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(proxy_offsets_kernel, dim3(1), dim3(1024), 0, st, k, kappa, T, k_max, m, N, tok_off, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || T == 0) return err;
  const int64_t A = (int64_t)T * m;
  hipLaunchKernelGGL(proxy_holes_kernel, dim3((unsigned)((A + 255) / 256)), dim3(256), 0, st, k, kappa, T, k_max, m, N,
                     base_tok_off, base_ids, E_base, tok_off, ids, wts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // blocks of the base permutation: at most A / 64 + min(E_base, A) for A = T * m rows
  const int64_t nblk = A / PX_ROWS + std::min<int64_t>(E_base, A);
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  const size_t lds = (size_t)PX_ROWS * N * sizeof(double);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(proxy_block_kernel<bf16_t>, grid, dim3(256), lds, st, k, kappa, k_max, m, N, r, Ip, base_tok_off,
                       base_w, base_eoff, base_ptok, base_psrc, (const bf16_t*)x, (const bf16_t*)wpg,
                       (const bf16_t*)wpu, E_base, d, blocked, tok_off, ids, wts);
  else
    hipLaunchKernelGGL(proxy_block_kernel<float>, grid, dim3(256), lds, st, k, kappa, k_max, m, N, r, Ip, base_tok_off,
                       base_w, base_eoff, base_ptok, base_psrc, (const float*)x, (const float*)wpg, (const float*)wpu,
                       E_base, d, blocked, tok_off, ids, wts);
  return hipGetLastError();
}

}  // namespace moe
