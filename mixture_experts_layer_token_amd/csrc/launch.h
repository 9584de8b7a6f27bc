// Internal launchers of the MoE kernels (not exported).  Each enqueues its
// kernels on `st` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

enum { DT_F32 = 0, DT_BF16 = 1 };
constexpr int32_t MOE_DEV_BAD_K_BIT = 1;

// Budget each token executes (values of moe_k_policy): the validated k_t
// (EXACT), the batch maximum of the validated budgets for every valid token
// (BATCH_MAX), or k_t rounded up to a multiple of `granule` (ROUND_UP).
enum { K_EXACT = 0, K_BATCH_MAX = 1, K_ROUND_UP = 2 };
struct BudgetPolicy {
  int policy;
  int granule;
};

// route.hip
// K slices of the router (float64 partial sums part[S][T][E]); depends on the shape only.
int router_splits(int T, int d, int E);
// Router partial logits; also writes tok_off and status (token-offset scan).
hipError_t launch_router(int dtype, const void* x, const void* w, const int32_t* k, int T, int d, int E, int k_max,
                         BudgetPolicy pol, int S, double* part, int32_t* tok_off, int32_t* status, hipStream_t st);
// Sums the S slices in order, adds the bias, rounds to float32, selects top-k_t.
hipError_t launch_topk(const double* part, int S, const float* bias, const int32_t* tok_off, int T, int E,
                       int k_max, float scale, int32_t* ids, float* wts, hipStream_t st);
// Small batches in one launch (one workgroup per token, float64 over the whole
// d): offsets, status, ids and weights as launch_router + launch_topk.
int fused_router_ok(int T, int d, int E);
int fused_router_auto(int T, int d, int E);
hipError_t launch_router_fused(int dtype, const void* x, const void* w, const float* bias, const int32_t* k, int T,
                               int d, int E, int k_max, BudgetPolicy pol, float scale, int32_t* tok_off,
                               int32_t* status, int32_t* ids, float* wts, hipStream_t st);

// route_screen.hip -- bf16 only: MFMA logits with an error bound screen the
// candidates; exact fp64 logits for candidates; same selection and weights.
// K slices of the screening pass (partials approx, absum: float [S][T][E]).
int router_screen_splits(int T, int d, int E);
// Token offsets (first workgroup), screening pass, then selection.
hipError_t launch_router_screen(const void* x, const void* w, const float* bias, const int32_t* k, int T, int d,
                                int E, int k_max, BudgetPolicy pol, int S, float scale, float* approx, float* absum,
                                int32_t* tok_off, int32_t* status, int32_t* ids, float* wts, hipStream_t st);

// Row-block table of the grouped FFN kernels.  The rows of group g,
// [grp_off[g], grp_off[g+1]), are cut into blocks of RB rows; entry i is
// {g, first row, rows in the block, 0} for i < count, {-1, 0, 0, 0} for
// count <= i < bound, and entry `bound` is {count, 0, 0, 0}.  `bound` comes
// from the shape only (it sizes launch grids): sum_g ceil(rows_g / RB) <=
// A_cap / RB + min(G, A_cap) when sum_g rows_g <= A_cap.
int row_block_bound(int A_cap, int G, int RB);
// One workgroup (G <= 1024) builds the table from grp_off.
hipError_t launch_row_blocks(const int32_t* grp_off, int G, int RB, int bound, int4* blocks, hipStream_t st);

// permute.hip
constexpr int PERM_BLOCK = 256;  // tokens per histogram block
// blocks (nullable): also writes the row-block table of the expert groups
// (RB rows per block, `bound` entries + the count), as launch_row_blocks would.
hipError_t launch_permute(const int32_t* tok_off, const int32_t* ids, int T, int E, int k_max, int32_t* block_counts,
                          int32_t* block_base, int32_t* counts, int32_t* expert_off, int32_t* perm_tok,
                          int32_t* perm_src, int32_t* inv_perm, int32_t* n_active, int32_t* stats, int RB,
                          int bound, int4* blocks, hipStream_t st);

// ffn_stream.hip -- weight-streaming grouped FFN.
// A second, dense problem of the same N and K that a routed FFN launch (either
// path) can carry: rows [0, rows) of `in` (no row map) against weights w0 / w1
// into `out` -- the always-on shared expert.  In the grouped GEMM its tiles
// come after the routed ones in each XCD's range in the gate/up launch
// (compute-bound tiles that fill the CUs the end of the weight stream leaves
// idle) and before them in the down launch (short tiles); in the streaming
// kernel its blocks come first (they are that launch's longest items).
struct GemmSecond {
  const void* in = nullptr;
  const void* w0 = nullptr;
  const void* w1 = nullptr;
  void* out = nullptr;
  int rows = 0;
};

//  gate/up: H[r] = SiLU(in[src(r)] . wg[g]^T) * (in[src(r)] . wu[g]^T), N = I, K = d
//  down:    Y[r] = H[r] . wd[g]^T,                                     N = d, K = I
// Work: the row-block table `blocks` (RB = stream_row_block(), `bound` entries)
// of the expert groups; blocks == nullptr means one dense group of
// `dense_rows` rows starting at 0 (weights of group 0).  src(r) = row_map[r]
// when row_map != nullptr, else r.  `blocked`: the weights are stored in the
// blocked order of w_offset (common.h), else row-major.
int stream_row_block();
hipError_t launch_ffn_gateup_stream(int dtype, const void* in, const int32_t* row_map, const void* wg,
                                    const void* wu, const int4* blocks, int bound, int dense_rows, void* h, int N,
                                    int K, int blocked, hipStream_t st, const GemmSecond& sec = GemmSecond{});
hipError_t launch_ffn_down_stream(int dtype, const void* h, const int32_t* row_map, const void* wd,
                                  const int4* blocks, int bound, int dense_rows, void* y, int N, int K, int blocked,
                                  hipStream_t st, const GemmSecond& sec = GemmSecond{});

// ffn_gemm.hip -- grouped-GEMM FFN (bf16): same semantics as the streaming
// kernels, over the row-block table with RB = gemm_row_block(rows_hint) (`bound`
// entries + count; blocks == nullptr: one dense group of dense_rows rows).
// rows_hint (an estimate of rows per group, from the shape only) picks the
// tile height.  N must be a multiple of 128 and K of 64.  `sec`: the second,
// dense problem above.
int gemm_row_block(int rows_hint);
hipError_t launch_ffn_gateup_gemm(const void* in, const int32_t* row_map, const void* wg, const void* wu,
                                  const int4* blocks, int bound, int dense_rows, int rows_hint, void* h, int N,
                                  int K, int blocked, hipStream_t st, const GemmSecond& sec = GemmSecond{});
hipError_t launch_ffn_down_gemm(const void* h, const int32_t* row_map, const void* wd, const int4* blocks, int bound,
                                int dense_rows, int rows_hint, void* y, int N, int K, int blocked, hipStream_t st,
                                const GemmSecond& sec = GemmSecond{});

// layout.hip -- row-major -> blocked copy of G [N][K] matrices (w_offset).
hipError_t launch_pack_weights(int dtype, long long G, int N, int K, const void* src, void* dst, hipStream_t st);

// combine.hip -- k_max (the largest budget) sets how many rows a thread
// requests at once.
hipError_t launch_combine(int dtype, const void* y, const void* y_shared, const int32_t* tok_off,
                          const float* wts, const int32_t* inv_perm, void* out, int T, int d, int k_max,
                          hipStream_t st);

// fold.hip -- expert folding of the routing metadata.  mode 0: keep at most
// `budget` routes per token; mode 1: keep a pool of `budget` experts (needs
// expert_off / perm_src of the input routes).  Scratch: ids / w [T * k_max]
// (folded routes at the input offsets), cnt [T], pool / members [E],
// n_members [1].  k_t <= 64.
struct FoldScratch {
  int32_t* ids;
  float* w;
  int32_t* cnt;
  int32_t* pool;
  int32_t* members;
  int32_t* n_members;
};
hipError_t launch_fold(int mode, int budget, const float* S, const float* L, const float* H, const int32_t* tok_off,
                       const int32_t* ids, const float* w, const int32_t* expert_off, const int32_t* perm_src, int T,
                       int E, int32_t* tok_off_out, int32_t* ids_out, float* w_out, int32_t* pool_out,
                       const FoldScratch& ws, hipStream_t st);

// proxy.hip -- training-free proxy gating of a split layer.
hipError_t launch_proxy_pack(int dtype, const int32_t* gate_idx, const void* wg, const void* wu, int E_base, int I_sub,
                             int d, int N, int r, int Ip, void* pg, void* pu, int blocked, hipStream_t st);
hipError_t launch_proxy_route(int dtype, const int32_t* k, const int32_t* kappa, int T, int k_max, int m, int N, int r,
                              int Ip, const int32_t* base_tok_off, const int32_t* base_ids, const float* base_w,
                              const int32_t* base_eoff, const int32_t* base_ptok, const int32_t* base_psrc,
                              const void* x, const void* wpg, const void* wpu, int E_base, int d, int blocked,
                              int32_t* tok_off, int32_t* ids, float* wts, int32_t* status, hipStream_t st);

// path.hip -- compositional path routing (PCoMoE).  `table`: int32 src[P],
// int32 tgt[P], float bias[P].
// The screened router's MFMA pass alone (partials and the token scan).
hipError_t launch_router_screen_partials(const void* x, const void* w, const int32_t* k, int T, int d, int E,
                                         int k_max, BudgetPolicy pol, int S, float* approx, float* absum,
                                         int32_t* tok_off, int32_t* status, hipStream_t st);
// Screened path selection (bf16, E <= 256): MFMA-pass bounds on every path
// score, exact logits only for the sources and targets of the candidates.
hipError_t launch_path_screen(const void* x, const void* w_router, const void* w_tgt, const float* bias,
                              const float* ag, const float* sg, const float* at, const float* st_, int S,
                              const void* table, int P, float lam, const int32_t* tok_off, int T, int d, int E,
                              int k_max, float scale, int32_t* osrc, int32_t* otgt, float* wts, hipStream_t st);
hipError_t launch_path_topk(const double* part_g, const double* part_t, int S, const float* bias,
                            const void* table, int P, float lam, const int32_t* tok_off, int T, int E, int k_max,
                            float scale, int32_t* osrc, int32_t* otgt, float* wts, hipStream_t st);
hipError_t launch_path_sources(const int32_t* tok_off, const int32_t* psrc, int T, int E, int k_max, int32_t* cnt,
                               int32_t* tmp, int32_t* src_off, int32_t* src_ids, int32_t* p2s, int32_t* unit_off,
                               hipStream_t st);
hipError_t launch_path_rows(const int32_t* tok_off, int T, int k_max, const int32_t* perm_path, const int32_t* p2s,
                            const int32_t* src_inv, int32_t* row_map, hipStream_t st);

// moe_abi.cpp -- the forward of moe_forward over a caller-chosen scratch
// region.  own_regions: `ws` holds only the forward's own regions
// (forward_scratch_bytes), as the no-allocation entry point supplies;
// otherwise the moe_workspace_size(MOE_OP_FORWARD) rule applies.
size_t forward_scratch_bytes(const moe_desc& d);
// Descriptor and path valid, and the forward's own regions fit in `capacity`
// bytes (else MOE_ERR_SCRATCH).
moe_status forward_scratch_check(const moe_desc* desc, size_t capacity);
moe_status forward_impl(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                        const int32_t* k, const void* w_gate, const void* w_up, const void* w_down,
                        const void* ws_gate, const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                        int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream, bool own_regions);

// probe.hip -- streaming-read probe (measurement only): reads `bytes` of src
// once (16-byte loads, non-temporal if asked); sink receives at most 4 bytes.
hipError_t launch_read_probe(const void* src, size_t bytes, int nontemporal, uint32_t* sink, hipStream_t st);

}  // namespace moe
