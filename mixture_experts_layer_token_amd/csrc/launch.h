// Internal launchers of the MoE kernels (not exported).  Each enqueues its
// kernels on `st` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { DT_F32 = 0, DT_BF16 = 1 };
constexpr int32_t MOE_DEV_BAD_K_BIT = 1;

// route.hip
// K slices of the router (float64 partial sums part[S][T][E]); depends on the shape only.
int router_splits(int T, int d, int E);
// Router partial logits; also writes tok_off and status (token-offset scan).
hipError_t launch_router(int dtype, const void* x, const void* w, const int32_t* k, int T, int d, int E, int k_max,
                         int S, double* part, int32_t* tok_off, int32_t* status, hipStream_t st);
// Sums the S slices in order, adds the bias, rounds to float32, selects top-k_t.
hipError_t launch_topk(const double* part, int S, const float* bias, const int32_t* tok_off, int T, int E,
                       float scale, int32_t* ids, float* wts, hipStream_t st);
// Token offsets alone (one workgroup).
hipError_t launch_tok_offsets(const int32_t* k, int T, int k_max, int32_t* tok_off, int32_t* status, hipStream_t st);

// route_screen.hip -- bf16 only: MFMA logits with an error bound screen the
// candidates; exact fp64 logits for candidates; same selection and weights.
// approx, absum: float [T][E] scratch.  tok_off must be ready.
hipError_t launch_router_screen(const void* x, const void* w, const float* bias, const int32_t* tok_off, int T,
                                int d, int E, float scale, float* approx, float* absum, int32_t* ids, float* wts,
                                hipStream_t st);

// permute.hip
constexpr int PERM_BLOCK = 256;  // tokens per histogram block
hipError_t launch_permute(const int32_t* tok_off, const int32_t* ids, int T, int E, int32_t* block_counts,
                          int32_t* block_base, int32_t* counts, int32_t* expert_off, int32_t* perm_tok,
                          int32_t* perm_src, int32_t* inv_perm, int32_t* n_active, int32_t* stats,
                          hipStream_t st);

// ffn_stream.hip -- weight-streaming grouped FFN.
//  gate/up: H[row0+m] = SiLU(in[src(m)] . wg[g]^T) * (in[src(m)] . wu[g]^T), N = I, K = d
//  down:    Y[row0+m] = H[row0+m] . wd[g]^T,                                 N = d, K = I
// Groups: G experts with rows [grp_off[g], grp_off[g+1]); grp_off == nullptr
// means one group of `dense_rows` rows starting at 0.  src(m) = row_map[row0+m]
// when row_map != nullptr, else row0 + m.  rows_max bounds the rows of any
// group (it sizes the grid; it must not depend on the routing).
hipError_t launch_ffn_gateup_stream(int dtype, const void* in, const int32_t* row_map, const void* wg,
                                    const void* wu, const int32_t* grp_off, int G, int dense_rows, int rows_max,
                                    void* h, int N, int K, hipStream_t st);
hipError_t launch_ffn_down_stream(int dtype, const void* h, const void* wd, const int32_t* grp_off, int G,
                                  int dense_rows, int rows_max, void* y, int N, int K, hipStream_t st);

// ffn_gemm.hip -- grouped-GEMM FFN (bf16): same semantics as the streaming
// kernels.  tile_off [G+1] (row blocks of 256 per group) is built on the device
// by launch_gemm_tiles; rb_bound >= tile_off[G] sizes the grid and rows_hint
// (an estimate of rows per group) picks the tile height -- both from the shape
// only.  N must be a multiple of 128 and K of 64.
int gemm_tile_bound(int A_cap, int G);
hipError_t launch_gemm_tiles(const int32_t* grp_off, int G, int32_t* tile_off, hipStream_t st);
hipError_t launch_ffn_gateup_gemm(const void* in, const int32_t* row_map, const void* wg, const void* wu,
                                  const int32_t* grp_off, const int32_t* tile_off, int G, int dense_rows,
                                  int rb_bound, int rows_hint, void* h, int N, int K, hipStream_t st);
hipError_t launch_ffn_down_gemm(const void* h, const void* wd, const int32_t* grp_off, const int32_t* tile_off,
                                int G, int dense_rows, int rb_bound, int rows_hint, void* y, int N, int K,
                                hipStream_t st);

// combine.hip
hipError_t launch_combine(int dtype, const void* y, const void* y_shared, const int32_t* tok_off,
                          const float* wts, const int32_t* inv_perm, void* out, int T, int d, hipStream_t st);

}  // namespace moe
