// Exported C ABI of the MoE layer library (declared in include/moe.h).
// Host-side validation, workspace planning and launch sequencing only; all
// arithmetic runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/moe.h"
#include "launch.h"

namespace {

using namespace moe;

constexpr int kDimQuantum = 128;  // d, I and I_shared must be multiples of this

size_t elt_size(const moe_desc& d) { return d.dtype == MOE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_GEMM) return MOE_ERR_UNSUPPORTED;
  if (d->router < MOE_ROUTER_AUTO || d->router > MOE_ROUTER_FUSED) return MOE_ERR_UNSUPPORTED;
  if (d->router == MOE_ROUTER_FUSED && !fused_router_ok(d->T, d->d, d->E)) return MOE_ERR_UNSUPPORTED;
  if (d->router == MOE_ROUTER_SCREENED && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->T < 0 || d->E < 1 || d->E > 1024 || d->k_max < 1 || d->k_max > d->E) return MOE_ERR_SHAPE;
  if (d->d < kDimQuantum || d->d > 65536 || d->d % kDimQuantum) return MOE_ERR_SHAPE;
  if (d->I < kDimQuantum || d->I > 65536 || d->I % kDimQuantum) return MOE_ERR_SHAPE;
  if (d->I_shared < 0 || d->I_shared > 65536 || d->I_shared % kDimQuantum) return MOE_ERR_SHAPE;
  if ((int64_t)d->T * d->k_max >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (!std::isfinite(d->routed_scale)) return MOE_ERR_SHAPE;
  if (d->k_policy < MOE_K_EXACT || d->k_policy > MOE_K_ROUND_UP) return MOE_ERR_UNSUPPORTED;
  if (d->k_policy == MOE_K_ROUND_UP && (d->k_granule < 1 || d->k_max % d->k_granule)) return MOE_ERR_SHAPE;
  if (d->weight_layout != MOE_W_ROWMAJOR && d->weight_layout != MOE_W_BLOCKED64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Carves 256-byte-aligned regions out of a workspace (or only sizes them when
// base == nullptr).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
  void* take_bytes(size_t n) { return take<char>(n); }
  size_t total() const { return (off + 255) & ~size_t(255); }
};

size_t a_cap(const moe_desc& d) { return (size_t)d.T * d.k_max; }
BudgetPolicy budget(const moe_desc& d) {
  return BudgetPolicy{d.k_policy, d.k_policy == MOE_K_ROUND_UP ? d.k_granule : 1};
}
int n_blocks(const moe_desc& d) { return (d.T + PERM_BLOCK - 1) / PERM_BLOCK; }

struct RouteWs { double* part; int splits; float* approx; float* absum; bool screened; bool fused; };
struct PermWs { int32_t* block_counts; int32_t* block_base; };
struct FfnWs { int4* blocks; int bound; int rb; void* h; void* h_sh; };

// Large bf16 batches route through the MFMA screen (exact on the candidates);
// smaller ones sum every logit in float64 directly.
bool screened_router(const moe_desc& d) {
  if (d.router == MOE_ROUTER_SCREENED) return true;
  if (d.router == MOE_ROUTER_FLOAT64 || d.router == MOE_ROUTER_FUSED) return false;
  return d.dtype == MOE_BF16 && (double)d.T * d.E * d.d >= 1073741824.0;
}
// Small batches with few router rows (T <= 1024, E <= 256, E * d <= 2^16)
// route in one launch under AUTO; MOE_ROUTER_FUSED asks for it up to 2^19.
bool fused_router(const moe_desc& d) {
  if (d.router == MOE_ROUTER_FUSED) return true;
  if (d.router != MOE_ROUTER_AUTO || screened_router(d)) return false;
  return fused_router_auto(d.T, d.d, d.E) != 0;
}

void plan_route(const moe_desc& d, Carver& c, RouteWs& w) {
  w.screened = screened_router(d);
  w.fused = fused_router(d);
  if (w.fused) {  // no partial sums
    w.part = nullptr;
    w.approx = w.absum = nullptr;
    w.splits = 0;
    return;
  }
  w.splits = w.screened ? router_screen_splits(d.T, d.d, d.E) : router_splits(d.T, d.d, d.E);
  const size_t ste = (size_t)w.splits * d.T * d.E;
  const size_t bytes = w.screened ? 2 * ste * sizeof(float) : ste * sizeof(double);
  char* p = static_cast<char*>(c.take_bytes(bytes));
  w.part = reinterpret_cast<double*>(p);
  w.approx = reinterpret_cast<float*>(p);
  w.absum = p ? reinterpret_cast<float*>(p + ste * sizeof(float)) : nullptr;
}
void plan_permute(const moe_desc& d, Carver& c, PermWs& w) {
  const size_t n = (size_t)n_blocks(d) * d.E;
  w.block_counts = c.take<int32_t>(n);
  w.block_base = c.take<int32_t>(n);
}
// Rows per entry of the routed FFN's row-block table: the GEMM's row block,
// or the streaming kernel's rows per workgroup.
bool routed_gemm(const moe_desc& d);
int rows_hint(const moe_desc& d);
int ffn_rb(const moe_desc& d) { return routed_gemm(d) ? gemm_row_block(rows_hint(d)) : stream_row_block(); }

void plan_ffn(const moe_desc& d, Carver& c, FfnWs& w) {
  w.rb = ffn_rb(d);
  w.bound = row_block_bound((int)a_cap(d), d.E, w.rb);
  w.blocks = c.take<int4>((size_t)w.bound + 1);
  w.h = c.take_bytes(a_cap(d) * d.I * elt_size(d));
  w.h_sh = d.I_shared ? c.take_bytes((size_t)d.T * d.I_shared * elt_size(d)) : nullptr;
}

struct FwdWs {
  RouteWs r;
  PermWs p;
  FfnWs f;
  int32_t *tok_off, *ids, *counts, *expert_off, *perm_tok, *perm_src, *inv_perm, *n_active, *status;
  float* w;
  void *y, *y_sh;
};

void plan_forward(const moe_desc& d, Carver& c, FwdWs& w) {
  plan_route(d, c, w.r);
  plan_permute(d, c, w.p);
  plan_ffn(d, c, w.f);
  const size_t A = a_cap(d);
  w.tok_off = c.take<int32_t>((size_t)d.T + 1);
  w.ids = c.take<int32_t>(A);
  w.w = c.take<float>(A);
  w.counts = c.take<int32_t>(d.E);
  w.expert_off = c.take<int32_t>((size_t)d.E + 1);
  w.perm_tok = c.take<int32_t>(A);
  w.perm_src = c.take<int32_t>(A);
  w.inv_perm = c.take<int32_t>(A);
  w.n_active = c.take<int32_t>(1);
  w.status = c.take<int32_t>(1);
  w.y = c.take_bytes(A * d.d * elt_size(d));
  w.y_sh = d.I_shared ? c.take_bytes((size_t)d.T * d.d * elt_size(d)) : nullptr;
}

void plan_fold(const moe_desc& d, Carver& c, FoldScratch& w) {
  const size_t A = a_cap(d);
  w.ids = c.take<int32_t>(A);
  w.w = c.take<float>(A);
  w.cnt = c.take<int32_t>((size_t)d.T);
  w.pool = c.take<int32_t>(d.E);
  w.members = c.take<int32_t>(d.E);
  w.n_members = c.take<int32_t>(1);
}

// Path routing: the screened selection (MFMA bounds, exact logits for the
// candidates' sources and targets) where the router would screen and E <= 256;
// otherwise every logit in float64.
struct PathWs {
  bool screened;
  int splits;
  double *part_g, *part_t;     // float64 partials (unscreened)
  float *ag, *sg, *at, *st;    // MFMA partials and |x||w| sums (screened)
  int32_t *cnt, *tmp;
};
void plan_path(const moe_desc& d, Carver& c, PathWs& w) {
  w.screened = d.E <= 256 && screened_router(d);
  w.splits = w.screened ? router_screen_splits(d.T, d.d, d.E) : router_splits(d.T, d.d, d.E);
  const size_t ste = (size_t)w.splits * d.T * d.E;
  w.part_g = w.part_t = nullptr;
  w.ag = w.sg = w.at = w.st = nullptr;
  if (w.screened) {
    w.ag = c.take<float>(ste);
    w.sg = c.take<float>(ste);
    w.at = c.take<float>(ste);
    w.st = c.take<float>(ste);
  } else {
    w.part_g = c.take<double>(ste);
    w.part_t = c.take<double>(ste);
  }
  w.cnt = c.take<int32_t>((size_t)d.T);
  w.tmp = c.take<int32_t>(a_cap(d));
}

size_t ws_size(const moe_desc& d, int op) {
  Carver c(nullptr);
  switch (op) {
    case MOE_OP_ROUTE: { RouteWs w; plan_route(d, c, w); break; }
    case MOE_OP_PERMUTE: { PermWs w; plan_permute(d, c, w); break; }
    case MOE_OP_FFN: { FfnWs w; plan_ffn(d, c, w); break; }
    case MOE_OP_COMBINE: break;
    case MOE_OP_FOLD: { FoldScratch w; plan_fold(d, c, w); break; }
    case MOE_OP_PATH: { PathWs w; plan_path(d, c, w); break; }
    default: {  // the forward's own regions; large enough for every other op
      FwdWs w;
      plan_forward(d, c, w);
      Carver f(nullptr), p(nullptr);
      FoldScratch fw;
      plan_fold(d, f, fw);
      PathWs pw;
      plan_path(d, p, pw);
      return std::max({c.total(), f.total(), p.total()});
    }
  }
  return c.total();
}

// Token-indexed buffers may be NULL when there are no tokens (empty tensors).
bool tok_ptr(const moe_desc& d, const void* p) { return p != nullptr || d.T == 0; }

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

#define MOE_TRY(expr)                              \
  do {                                             \
    moe_status s_ = (expr);                        \
    if (s_ != MOE_OK) return s_;                   \
  } while (0)

moe_status check_ws(const moe_desc& d, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_size(d, op);
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status path_ok(const moe_desc& d) {
  // The grouped GEMM is a bf16 kernel.
  return (d.path == MOE_PATH_GEMM && d.dtype != MOE_BF16) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

// Path choice.  Rows per expert set the roofline: a few rows per expert make the
// FFN a weight stream (HBM-bound), hundreds make it a dense contraction.  AUTO
// takes the grouped GEMM when the bound on assignments per expert,
// T * k_max / E, reaches 64 (shape only, so the choice never depends on routing).
bool routed_gemm(const moe_desc& d) {
  if (d.dtype != MOE_BF16 || d.path == MOE_PATH_STREAM) return false;
  if (d.path == MOE_PATH_GEMM) return true;
  return (int64_t)d.T * d.k_max >= (int64_t)64 * d.E;
}
// Rows-per-expert estimate for the GEMM tile choice: the bound T * k_max / E
// (shape only).
int rows_hint(const moe_desc& d) { return (int)std::min<int64_t>((int64_t)d.T * d.k_max / d.E, d.T); }
bool shared_gemm(const moe_desc& d) {
  if (d.dtype != MOE_BF16 || d.path == MOE_PATH_STREAM) return false;
  return d.path == MOE_PATH_GEMM || d.T >= 256;
}
// The shared expert runs inside the routed grouped-GEMM launches (its row
// tiles interleaved with the routed ones) when both take the GEMM path and
// its intermediate size equals the routed one.
// The shared expert rides in the routed FFN launches (as their last tiles)
// when it is as wide as a routed expert and both take the same path.
bool fused_shared(const moe_desc& d) {
  return d.I_shared > 0 && d.I_shared == d.I && routed_gemm(d) == shared_gemm(d);
}

// ---- stage bodies (arguments already validated) ----

moe_status do_route(const moe_desc& d, const void* x, const void* wr, const float* bias, const int32_t* k,
                    int32_t* tok_off, int32_t* ids, float* w, int32_t* status, const RouteWs& ws, hipStream_t st) {
  if (ws.fused)
    return launched(launch_router_fused(d.dtype, x, wr, bias, k, d.T, d.d, d.E, d.k_max, budget(d), d.routed_scale,
                                        tok_off, status, ids, w, st));
  if (ws.screened)
    return launched(launch_router_screen(x, wr, bias, k, d.T, d.d, d.E, d.k_max, budget(d), ws.splits, d.routed_scale,
                                         ws.approx,
                                         ws.absum, tok_off, status, ids, w, st));
  hipError_t e =
      launch_router(d.dtype, x, wr, k, d.T, d.d, d.E, d.k_max, budget(d), ws.splits, ws.part, tok_off, status, st);
  if (e == hipSuccess) e = launch_topk(ws.part, ws.splits, bias, tok_off, d.T, d.E, d.k_max, d.routed_scale, ids, w, st);
  return launched(e);
}

moe_status do_permute(const moe_desc& d, const int32_t* tok_off, const int32_t* ids, int32_t* counts,
                      int32_t* expert_off, int32_t* perm_tok, int32_t* perm_src, int32_t* inv_perm,
                      int32_t* n_active, int32_t* stats, const PermWs& ws, const FfnWs* fw, hipStream_t st) {
  return launched(launch_permute(tok_off, ids, d.T, d.E, d.k_max, ws.block_counts, ws.block_base, counts, expert_off,
                                 perm_tok, perm_src, inv_perm, n_active, stats, fw ? fw->rb : 1, fw ? fw->bound : 0,
                                 fw ? fw->blocks : nullptr, st));
}

// The row-block table fw.blocks is built here when `build_blocks` (otherwise
// the permutation wrote it).
// `sec`: the shared expert's part when it is fused into the routed launch.
moe_status do_gateup(const moe_desc& d, const void* x, const void* wg, const void* wu, const int32_t* expert_off,
                     const int32_t* perm_tok, void* h, const FfnWs& fw, bool build_blocks, hipStream_t st,
                     const GemmSecond& sec = GemmSecond{}) {
  hipError_t e = build_blocks ? launch_row_blocks(expert_off, d.E, fw.rb, fw.bound, fw.blocks, st) : hipSuccess;
  if (e != hipSuccess) return launched(e);
  if (routed_gemm(d))
    return launched(
        launch_ffn_gateup_gemm(x, perm_tok, wg, wu, fw.blocks, fw.bound, 0, rows_hint(d), h, d.I, d.d, d.weight_layout, st,
                               sec));
  return launched(launch_ffn_gateup_stream(d.dtype, x, perm_tok, wg, wu, fw.blocks, fw.bound, 0, h, d.I, d.d,
                                           d.weight_layout, st, sec));
}

// `row_map`: the h row of each permuted row (NULL: row p reads h row p).
moe_status do_down(const moe_desc& d, const void* h, const void* wd, const int32_t* expert_off, void* y,
                   const FfnWs& fw, bool build_blocks, hipStream_t st, const GemmSecond& sec = GemmSecond{},
                   const int32_t* row_map = nullptr) {
  hipError_t e = build_blocks ? launch_row_blocks(expert_off, d.E, fw.rb, fw.bound, fw.blocks, st) : hipSuccess;
  if (e != hipSuccess) return launched(e);
  if (routed_gemm(d))
    return launched(launch_ffn_down_gemm(h, row_map, wd, fw.blocks, fw.bound, 0, rows_hint(d), y, d.d, d.I,
                                              d.weight_layout, st, sec));
  return launched(launch_ffn_down_stream(d.dtype, h, row_map, wd, fw.blocks, fw.bound, 0, y, d.d, d.I, d.weight_layout, st,
                                         sec));
}

moe_status do_shared(const moe_desc& d, const void* x, const void* sg, const void* su, const void* sd, void* h_sh,
                     void* y_sh, hipStream_t st) {
  hipError_t e;
  if (shared_gemm(d)) {
    e = launch_ffn_gateup_gemm(x, nullptr, sg, su, nullptr, 0, d.T, d.T, h_sh, d.I_shared, d.d, d.weight_layout, st);
    if (e == hipSuccess)
      e = launch_ffn_down_gemm(h_sh, nullptr, sd, nullptr, 0, d.T, d.T, y_sh, d.d, d.I_shared, d.weight_layout, st);
    return launched(e);
  }
  e = launch_ffn_gateup_stream(d.dtype, x, nullptr, sg, su, nullptr, 0, d.T, h_sh, d.I_shared, d.d, d.weight_layout, st);
  if (e == hipSuccess)
    e = launch_ffn_down_stream(d.dtype, h_sh, nullptr, sd, nullptr, 0, d.T, y_sh, d.d, d.I_shared, d.weight_layout,
                                   st);
  return launched(e);
}

moe_status do_combine(const moe_desc& d, const void* y, const void* y_sh, const int32_t* tok_off, const float* w,
                      const int32_t* inv_perm, void* out, hipStream_t st) {
  return launched(launch_combine(d.dtype, y, y_sh, tok_off, w, inv_perm, out, d.T, d.d, d.k_max, st));
}

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_desc* desc, int32_t op, size_t* bytes) {
  MOE_TRY(check_desc(desc));
  if (!bytes) return MOE_ERR_NULL;
  if (op < MOE_OP_ROUTE || op > MOE_OP_PATH) return MOE_ERR_UNSUPPORTED;
  *bytes = ws_size(*desc, op);
  return MOE_OK;
}

moe_status moe_pack_weights(int32_t dtype, int32_t G, int32_t N, int32_t K, const void* src, void* dst,
                            moe_stream_t stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int elt = dtype == MOE_BF16 ? 2 : 4, eb = 128 / elt;
  if (G < 0 || N < 1 || K < 1 || N % 64 || K % eb) return MOE_ERR_SHAPE;
  const long long n = (long long)G * N * K;
  if (n >= (1ll << 40)) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t bytes = (uintptr_t)n * elt;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_SHAPE;
  return launched(launch_pack_weights(dtype, G, N, K, src, dst, static_cast<hipStream_t>(stream)));
}

moe_status moe_resolve_path(const moe_desc* desc, int32_t* routed_path, int32_t* shared_path) {
  MOE_TRY(check_desc(desc));
  if (!routed_path || !shared_path) return MOE_ERR_NULL;
  MOE_TRY(path_ok(*desc));
  *routed_path = routed_gemm(*desc) ? MOE_PATH_GEMM : MOE_PATH_STREAM;
  *shared_path = shared_gemm(*desc) ? MOE_PATH_GEMM : MOE_PATH_STREAM;
  return MOE_OK;
}

moe_status moe_route(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                     const int32_t* k, int32_t* tok_off, int32_t* topk_ids, float* topk_w, int32_t* dev_status,
                     void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (!tok_ptr(d, x) || !w_router || !tok_ptr(d, k) || !tok_off || !tok_ptr(d, topk_ids) || !tok_ptr(d, topk_w))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(d, MOE_OP_ROUTE, ws, ws_bytes));
  Carver c(ws);
  RouteWs rw;
  plan_route(d, c, rw);
  return do_route(d, x, w_router, router_bias, k, tok_off, topk_ids, topk_w, dev_status, rw,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_desc* desc, const int32_t* tok_off, const int32_t* topk_ids,
                       int32_t* expert_counts, int32_t* expert_off, int32_t* perm_tok, int32_t* perm_src,
                       int32_t* inv_perm, int32_t* n_active, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (!tok_off || !tok_ptr(d, topk_ids) || !expert_counts || !expert_off || !tok_ptr(d, perm_tok) ||
      !tok_ptr(d, perm_src) || !tok_ptr(d, inv_perm) || !n_active)
    return MOE_ERR_NULL;
  MOE_TRY(check_ws(d, MOE_OP_PERMUTE, ws, ws_bytes));
  Carver c(ws);
  PermWs pw;
  plan_permute(d, c, pw);
  return do_permute(d, tok_off, topk_ids, expert_counts, expert_off, perm_tok, perm_src, inv_perm, n_active,
                    nullptr, pw, nullptr, static_cast<hipStream_t>(stream));
}

moe_status moe_ffn_plan(const moe_desc* desc, const int32_t* expert_off, void* ws, size_t ws_bytes,
                        moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  MOE_TRY(check_ws(d, MOE_OP_FFN, ws, ws_bytes));
  if (!expert_off) return MOE_ERR_NULL;
  Carver c(ws);
  FfnWs fw;
  plan_ffn(d, c, fw);
  return launched(launch_row_blocks(expert_off, d.E, fw.rb, fw.bound, fw.blocks, static_cast<hipStream_t>(stream)));
}

moe_status moe_ffn_gateup(const moe_desc* desc, const void* x, const void* w_gate, const void* w_up,
                          const int32_t* expert_off, const int32_t* perm_tok, void* h, void* ws, size_t ws_bytes,
                          moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  MOE_TRY(check_ws(d, MOE_OP_FFN, ws, ws_bytes));
  if (!tok_ptr(d, x) || !w_gate || !w_up || !expert_off || !tok_ptr(d, perm_tok) || !tok_ptr(d, h))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(h)) return MOE_ERR_ALIGN;
  Carver c(ws);
  FfnWs fw;
  plan_ffn(d, c, fw);
  return do_gateup(d, x, w_gate, w_up, expert_off, perm_tok, h, fw, false, static_cast<hipStream_t>(stream));
}

moe_status moe_ffn_down(const moe_desc* desc, const void* h, const void* w_down, const int32_t* expert_off,
                        void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  MOE_TRY(check_ws(d, MOE_OP_FFN, ws, ws_bytes));
  if (!tok_ptr(d, h) || !w_down || !expert_off || !tok_ptr(d, y_perm)) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(y_perm)) return MOE_ERR_ALIGN;
  Carver c(ws);
  FfnWs fw;
  plan_ffn(d, c, fw);
  return do_down(d, h, w_down, expert_off, y_perm, fw, false, static_cast<hipStream_t>(stream));
}

moe_status moe_ffn(const moe_desc* desc, const void* x, const void* w_gate, const void* w_up, const void* w_down,
                   const void* ws_gate, const void* ws_up, const void* ws_down, const int32_t* expert_off,
                   const int32_t* perm_tok, void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                   moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  if (!tok_ptr(d, x) || !w_gate || !w_up || !w_down || !expert_off || !tok_ptr(d, perm_tok) ||
      !tok_ptr(d, y_perm))
    return MOE_ERR_NULL;
  if (d.I_shared && (!ws_gate || !ws_up || !ws_down || !tok_ptr(d, y_shared))) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(y_perm))
    return MOE_ERR_ALIGN;
  if (d.I_shared && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(ws_down) || !aligned16(y_shared)))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(d, MOE_OP_FFN, ws, ws_bytes));
  Carver c(ws);
  FfnWs fw;
  plan_ffn(d, c, fw);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused_shared(d)) {
    MOE_TRY(do_gateup(d, x, w_gate, w_up, expert_off, perm_tok, fw.h, fw, true, st,
                      GemmSecond{x, ws_gate, ws_up, fw.h_sh, d.T}));
    return do_down(d, fw.h, w_down, expert_off, y_perm, fw, false, st,
                   GemmSecond{fw.h_sh, ws_down, ws_down, y_shared, d.T});
  }
  MOE_TRY(do_gateup(d, x, w_gate, w_up, expert_off, perm_tok, fw.h, fw, true, st));
  MOE_TRY(do_down(d, fw.h, w_down, expert_off, y_perm, fw, false, st));
  if (d.I_shared) MOE_TRY(do_shared(d, x, ws_gate, ws_up, ws_down, fw.h_sh, y_shared, st));
  return MOE_OK;
}

moe_status moe_combine(const moe_desc* desc, const void* y_perm, const void* y_shared, const int32_t* tok_off,
                       const float* topk_w, const int32_t* inv_perm, void* out, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (!tok_ptr(d, y_perm) || !tok_off || !tok_ptr(d, topk_w) || !tok_ptr(d, inv_perm) || !tok_ptr(d, out))
    return MOE_ERR_NULL;
  if (!aligned16(y_perm) || !aligned16(out) || (y_shared && !aligned16(y_shared))) return MOE_ERR_ALIGN;
  return do_combine(d, y_perm, y_shared, tok_off, topk_w, inv_perm, out, static_cast<hipStream_t>(stream));
}

moe_status moe_fold(const moe_desc* desc, int32_t mode, int32_t budget, const float* S, const float* L,
                    const float* H, const int32_t* tok_off, const int32_t* topk_ids, const float* topk_w,
                    const int32_t* expert_off, const int32_t* perm_src, int32_t* tok_off_out,
                    int32_t* ids_out, float* w_out, int32_t* pool_out, void* ws, size_t ws_bytes,
                    moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (mode != MOE_FOLD_TOKEN && mode != MOE_FOLD_POOL) return MOE_ERR_UNSUPPORTED;
  if (budget < 1 || d.k_max > 64) return MOE_ERR_SHAPE;
  if (!S || !L || !H || !tok_off || !tok_off_out || !tok_ptr(d, topk_ids) || !tok_ptr(d, topk_w) ||
      !tok_ptr(d, ids_out) || !tok_ptr(d, w_out))
    return MOE_ERR_NULL;
  if (mode == MOE_FOLD_POOL && (!expert_off || !tok_ptr(d, perm_src))) return MOE_ERR_NULL;
  MOE_TRY(check_ws(d, MOE_OP_FOLD, ws, ws_bytes));
  Carver c(ws);
  FoldScratch fw;
  plan_fold(d, c, fw);
  return launched(launch_fold(mode, budget, S, L, H, tok_off, topk_ids, topk_w, expert_off, perm_src, d.T, d.E,
                              tok_off_out, ids_out, w_out, pool_out, fw, static_cast<hipStream_t>(stream)));
}

static int proxy_width(int32_t N, int32_t r) {
  return (int)(((int64_t)N * r + kDimQuantum - 1) / kDimQuantum * kDimQuantum);
}

static moe_status proxy_shape(const moe_desc& d, int32_t N, int32_t r, int32_t m) {
  if (N < 1 || r < 1 || r > d.I || m < 1 || d.E % N || (int64_t)m * N > 64 || m > d.E / N ||
      d.k_max > m * N || (int64_t)N * r > 65536)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status moe_proxy_kappa_balanced(int32_t k_max, int32_t m, int32_t N, int32_t* kappa) {
  if (!kappa) return MOE_ERR_NULL;
  if (m < 1 || N < 1 || k_max < 0 || (int64_t)k_max > (int64_t)m * N) return MOE_ERR_SHAPE;
  for (int32_t k = 0; k <= k_max; ++k)
    for (int32_t j = 0; j < m; ++j) kappa[(size_t)k * m + j] = k / m + (j < k % m ? 1 : 0);
  return MOE_OK;
}

moe_status moe_proxy_pack(const moe_desc* desc, int32_t N, int32_t r, const int32_t* gate_idx, const void* w_gate,
                          const void* w_up, void* wp_gate, void* wp_up, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (N < 1 || r < 1 || r > d.I || d.E % N || (int64_t)N * r > 65536) return MOE_ERR_SHAPE;
  if (!gate_idx || !w_gate || !w_up || !wp_gate || !wp_up) return MOE_ERR_NULL;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(wp_gate) || !aligned16(wp_up)) return MOE_ERR_ALIGN;
  return launched(launch_proxy_pack(d.dtype, gate_idx, w_gate, w_up, d.E / N, d.I, d.d, N, r, proxy_width(N, r),
                                    wp_gate, wp_up, d.weight_layout, static_cast<hipStream_t>(stream)));
}

moe_status moe_proxy_route(const moe_desc* desc, int32_t N, int32_t r, int32_t m, const int32_t* k,
                           const int32_t* kappa, const int32_t* base_tok_off, const int32_t* base_ids,
                           const float* base_w, const int32_t* base_expert_off, const int32_t* base_perm_tok,
                           const int32_t* base_perm_src, const void* x, const void* wp_gate, const void* wp_up,
                           int32_t* tok_off, int32_t* topk_ids, float* topk_w, int32_t* dev_status,
                           moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(proxy_shape(d, N, r, m));
  if (!kappa || !tok_off || !tok_ptr(d, k) || !tok_ptr(d, base_tok_off) || !tok_ptr(d, base_ids) ||
      !tok_ptr(d, base_w) || !base_expert_off || !tok_ptr(d, base_perm_tok) || !tok_ptr(d, base_perm_src) ||
      !tok_ptr(d, x) || !wp_gate || !wp_up || !tok_ptr(d, topk_ids) || !tok_ptr(d, topk_w))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(wp_gate) || !aligned16(wp_up)) return MOE_ERR_ALIGN;
  return launched(launch_proxy_route(d.dtype, k, kappa, d.T, d.k_max, m, N, r, proxy_width(N, r), base_tok_off,
                                     base_ids, base_w, base_expert_off, base_perm_tok, base_perm_src, x, wp_gate,
                                     wp_up, d.E / N, d.d, d.weight_layout, tok_off, topk_ids, topk_w, dev_status,
                                     static_cast<hipStream_t>(stream)));
}

static constexpr int32_t kMaxPaths = 1024;

moe_status moe_path_table_bytes(int32_t P, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  if (P < 1 || P > kMaxPaths) return MOE_ERR_SHAPE;
  *bytes = (size_t)P * 12;
  return MOE_OK;
}

moe_status moe_path_table(int32_t E, int32_t P, const int32_t* src, const int32_t* tgt, const float* bias,
                          void* table, size_t table_bytes, moe_stream_t stream) {
  if (!src || !tgt || !bias || !table) return MOE_ERR_NULL;
  if (E < 1 || E > 1024 || P < 1 || P > kMaxPaths || table_bytes < (size_t)P * 12) return MOE_ERR_SHAPE;
  if (!aligned16(table)) return MOE_ERR_ALIGN;
  for (int32_t p = 0; p < P; ++p) {
    if (src[p] < 0 || src[p] >= E || tgt[p] < 0 || tgt[p] >= E || !std::isfinite(bias[p])) return MOE_ERR_SHAPE;
    if (p > 0 && (int64_t)src[p] * E + tgt[p] <= (int64_t)src[p - 1] * E + tgt[p - 1]) return MOE_ERR_SHAPE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* dst = static_cast<char*>(table);
  hipError_t e = hipMemcpyAsync(dst, src, (size_t)P * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(dst + (size_t)P * 4, tgt, (size_t)P * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(dst + (size_t)P * 8, bias, (size_t)P * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return launched(e);
}

static moe_status path_shape(const moe_desc& d, int32_t P) {
  if (P < 1 || P > kMaxPaths || d.k_max > 64 || d.k_max > P) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status moe_path_route(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                          const void* w_tgt, float lambda, const void* table, int32_t P, const int32_t* k,
                          int32_t* tok_off, int32_t* path_src, int32_t* path_tgt, float* path_w,
                          int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_shape(d, P));
  if (!std::isfinite(lambda)) return MOE_ERR_SHAPE;
  if (!tok_ptr(d, x) || !w_router || !table || !tok_ptr(d, k) || !tok_off || !tok_ptr(d, path_src) ||
      !tok_ptr(d, path_tgt) || !tok_ptr(d, path_w))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || (w_tgt && !aligned16(w_tgt)) || !aligned16(table))
    return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(d, MOE_OP_PATH, ws, ws_bytes));
  Carver c(ws);
  PathWs pw;
  plan_path(d, c, pw);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pw.screened) {
    hipError_t e = launch_router_screen_partials(x, w_router, k, d.T, d.d, d.E, d.k_max, budget(d), pw.splits, pw.ag,
                                                 pw.sg, tok_off, dev_status, st);
    if (e == hipSuccess && w_tgt)
      e = launch_router_screen_partials(x, w_tgt, k, d.T, d.d, d.E, d.k_max, budget(d), pw.splits, pw.at, pw.st,
                                        tok_off, dev_status, st);
    if (e == hipSuccess)
      e = launch_path_screen(x, w_router, w_tgt, router_bias, pw.ag, pw.sg, pw.at, pw.st, pw.splits, table, P,
                             lambda, tok_off, d.T, d.d, d.E, d.k_max, d.routed_scale, path_src, path_tgt, path_w, st);
    return launched(e);
  }
  hipError_t e = launch_router(d.dtype, x, w_router, k, d.T, d.d, d.E, d.k_max, budget(d), pw.splits, pw.part_g,
                               tok_off, dev_status, st);
  if (e == hipSuccess && w_tgt)
    e = launch_router(d.dtype, x, w_tgt, k, d.T, d.d, d.E, d.k_max, budget(d), pw.splits, pw.part_t, tok_off,
                      dev_status, st);
  if (e == hipSuccess)
    e = launch_path_topk(pw.part_g, w_tgt ? pw.part_t : nullptr, pw.splits, router_bias, table, P, lambda, tok_off,
                         d.T, d.E, d.k_max, d.routed_scale, path_src, path_tgt, path_w, st);
  return launched(e);
}

moe_status moe_path_sources(const moe_desc* desc, const int32_t* tok_off, const int32_t* path_src,
                            int32_t* src_tok_off, int32_t* src_ids, int32_t* path_src_route, int32_t* unit_off,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (d.k_max > 64) return MOE_ERR_SHAPE;
  if (!tok_off || !tok_ptr(d, path_src) || !src_tok_off || !tok_ptr(d, src_ids) || !tok_ptr(d, path_src_route) ||
      !unit_off)
    return MOE_ERR_NULL;
  MOE_TRY(check_ws(d, MOE_OP_PATH, ws, ws_bytes));
  Carver c(ws);
  PathWs pw;
  plan_path(d, c, pw);
  return launched(launch_path_sources(tok_off, path_src, d.T, d.E, d.k_max, pw.cnt, pw.tmp, src_tok_off, src_ids,
                                      path_src_route, unit_off, static_cast<hipStream_t>(stream)));
}

moe_status moe_path_rows(const moe_desc* desc, const int32_t* tok_off, const int32_t* perm_path,
                         const int32_t* path_src_route, const int32_t* src_inv_perm, int32_t* row_map,
                         moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  if (!tok_off || !tok_ptr(d, perm_path) || !tok_ptr(d, path_src_route) || !tok_ptr(d, src_inv_perm) ||
      !tok_ptr(d, row_map))
    return MOE_ERR_NULL;
  return launched(launch_path_rows(tok_off, d.T, d.k_max, perm_path, path_src_route, src_inv_perm, row_map,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_ffn_down_rows(const moe_desc* desc, const void* h, const int32_t* row_map, const void* w_down,
                             const int32_t* expert_off, void* y_perm, void* ws, size_t ws_bytes,
                             moe_stream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  MOE_TRY(check_ws(d, MOE_OP_FFN, ws, ws_bytes));
  if (!tok_ptr(d, h) || !tok_ptr(d, row_map) || !w_down || !expert_off || !tok_ptr(d, y_perm)) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(y_perm)) return MOE_ERR_ALIGN;
  Carver c(ws);
  FfnWs fw;
  plan_ffn(d, c, fw);
  return do_down(d, h, w_down, expert_off, y_perm, fw, false, static_cast<hipStream_t>(stream), GemmSecond{},
                 row_map);
}

moe_status moe_forward(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                       const int32_t* k, const void* w_gate, const void* w_up, const void* w_down,
                       const void* ws_gate, const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                       int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return moe::forward_impl(desc, x, w_router, router_bias, k, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out,
                           stats, dev_status, ws, ws_bytes, stream, false);
}

moe_status moe_probe_read(const void* src, size_t bytes, int32_t nontemporal, int32_t* sink, moe_stream_t stream) {
  if (bytes >= 16 && (!src || !sink)) return MOE_ERR_NULL;
  if (!aligned16(src)) return MOE_ERR_ALIGN;
  return launched(launch_read_probe(src, bytes, nontemporal, reinterpret_cast<uint32_t*>(sink),
                                    static_cast<hipStream_t>(stream)));
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "descriptor values outside the supported range";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, path or op";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_ALIGN: return "buffer not aligned (16 bytes; workspace 256 bytes)";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_SCRATCH: return "the layer needs more scratch than the library-held array holds";
  }
  return "unknown status";
}

}  // extern "C"

namespace moe {

size_t forward_scratch_bytes(const moe_desc& d) {
  Carver c(nullptr);
  FwdWs w;
  plan_forward(d, c, w);
  return c.total();
}

moe_status forward_scratch_check(const moe_desc* desc, size_t capacity) {
  MOE_TRY(check_desc(desc));
  MOE_TRY(path_ok(*desc));
  return forward_scratch_bytes(*desc) > capacity ? MOE_ERR_SCRATCH : MOE_OK;
}

moe_status forward_impl(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                        const int32_t* k, const void* w_gate, const void* w_up, const void* w_down,
                        const void* ws_gate, const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                        int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream, bool own_regions) {
  MOE_TRY(check_desc(desc));
  const moe_desc& d = *desc;
  MOE_TRY(path_ok(d));
  if (!tok_ptr(d, x) || !w_router || !tok_ptr(d, k) || !w_gate || !w_up || !w_down || !tok_ptr(d, out))
    return MOE_ERR_NULL;
  if (d.I_shared && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(out))
    return MOE_ERR_ALIGN;
  if (d.I_shared && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(ws_down))) return MOE_ERR_ALIGN;
  if (own_regions) {
    // the forward's own regions only (the caller's array is not shared with the other ops)
    if (!ws) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (forward_scratch_bytes(d) > ws_bytes) return MOE_ERR_SCRATCH;
  } else {
    MOE_TRY(check_ws(d, MOE_OP_FORWARD, ws, ws_bytes));
  }
  Carver c(ws);
  FwdWs fw;
  plan_forward(d, c, fw);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* status = dev_status ? dev_status : fw.status;
  MOE_TRY(do_route(d, x, w_router, router_bias, k, fw.tok_off, fw.ids, fw.w, status, fw.r, st));
  MOE_TRY(do_permute(d, fw.tok_off, fw.ids, fw.counts, fw.expert_off, fw.perm_tok, fw.perm_src, fw.inv_perm,
                     fw.n_active, stats, fw.p, &fw.f, st));
  if (fused_shared(d)) {
    MOE_TRY(do_gateup(d, x, w_gate, w_up, fw.expert_off, fw.perm_tok, fw.f.h, fw.f, false, st,
                      GemmSecond{x, ws_gate, ws_up, fw.f.h_sh, d.T}));
    MOE_TRY(do_down(d, fw.f.h, w_down, fw.expert_off, fw.y, fw.f, false, st,
                    GemmSecond{fw.f.h_sh, ws_down, ws_down, fw.y_sh, d.T}));
  } else {
    MOE_TRY(do_gateup(d, x, w_gate, w_up, fw.expert_off, fw.perm_tok, fw.f.h, fw.f, false, st));
    MOE_TRY(do_down(d, fw.f.h, w_down, fw.expert_off, fw.y, fw.f, false, st));
    if (d.I_shared) MOE_TRY(do_shared(d, x, ws_gate, ws_up, ws_down, fw.f.h_sh, fw.y_sh, st));
  }
  return do_combine(d, fw.y, fw.y_sh, fw.tok_off, fw.w, fw.inv_perm, out, st);
}

}  // namespace moe
