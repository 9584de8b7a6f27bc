/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward with a per-token
 * routing top-k.
 *
 * The problem statement follows the pages: hidden states, a linear router,
 * stacked SwiGLU experts and an externally supplied per-token budget k_t
 * (MoE-Prism, arXiv 2510.19366, §I and §III-C1: each request carries its own
 * routing top-k target, counted in routed experts and excluding shared
 * experts, §II-B).  The forward is split into the steps a serving stack runs
 * between attention blocks:
 *
 *   moe_route    router logits, top-k_t selection, renormalised softmax weights
 *   moe_permute  per-expert histogram, exclusive scan, (expert, token) permutation
 *   moe_ffn      grouped SwiGLU expert FFN over the permuted rows (+ shared expert)
 *   moe_combine  routing-weight-scaled sum back to token order
 *   moe_forward  all of the above in one call
 *
 * Every entry point is asynchronous on the caller's stream, allocates nothing,
 * never synchronises and never reads device memory on the host.  Launch grids
 * depend only on the descriptor, never on the k values or on the routing, so a
 * captured HIP graph of any entry point replays correctly for any k vector
 * (MoE-Prism §III-D: k must not become a graph-specialisation dimension).
 *
 * Conventions shared by all entry points
 * --------------------------------------
 *  - Pointers are device pointers unless stated.  Tensors are dense and
 *    row-major.  Activation, weight, H, Y and out buffers must be 16-byte
 *    aligned.  The caller owns every buffer.
 *  - "ELT" is the element type chosen by desc->dtype: float (MOE_F32) or
 *    bfloat16 (MOE_BF16, raw 16-bit storage).  x, the router weight, all
 *    expert weights, H, Y and out use ELT; routing weights are float32;
 *    indices and counts are int32.
 *  - Weight layout is the [out, in] convention:
 *      w_router [E][d], w_gate [E][I][d], w_up [E][I][d], w_down [E][d][I],
 *      ws_gate [Is][d], ws_up [Is][d], ws_down [d][Is]  (Is = I_shared).
 *    The expert weights (every w_gate/w_up/w_down/ws_* argument, and the
 *    proxy weights of moe_proxy_pack) are stored either row-major or in the
 *    blocked order of desc->weight_layout; the router weights are always
 *    row-major.
 *  - A = sum_t k_t is the number of (token, expert) assignments.  Arrays
 *    indexed by assignment have capacity T * k_max entries; only the first A
 *    are written.
 *  - Return value: MOE_OK, or an error from host-side validation (nothing is
 *    launched then), or MOE_ERR_LAUNCH when a kernel launch failed.
 *  - Routing is bit-reproducible: logits are the float64 sum of the exact
 *    products, rounded once to float32; selection and order use the key
 *    (logit descending, expert index ascending).  -0.0 and +0.0 compare equal.
 *  - Calls on one stream are ordered; calls that share a workspace must not
 *    overlap in time.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* descriptor values outside the supported range */
  MOE_ERR_UNSUPPORTED = 3, /* unknown dtype / path / op */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  MOE_ERR_ALIGN = 5,       /* a buffer is not 16-byte aligned (workspace: 256) */
  MOE_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch */
  MOE_ERR_SCRATCH = 7      /* moe_forward_noalloc: the layer needs more scratch than the
                              library-held array holds (MOE_NOALLOC_SCRATCH_BYTES) */
} moe_status;

/* FFN execution path.  Both compute the same function. */
typedef enum {
  MOE_PATH_AUTO = 0,    /* weight streaming when rows per expert are few, else grouped GEMM */
  MOE_PATH_STREAM = 1,  /* weight-streaming MFMA kernels (memory-bound decode) */
  MOE_PATH_GEMM = 2     /* LDS-tiled grouped GEMM on MFMA (compute-bound prefill) */
} moe_path;

/* Router algorithm.  Both produce identical ids, order and weights (the
 * routing contract below); they differ only in cost. */
typedef enum {
  MOE_ROUTER_AUTO = 0,      /* screened for bf16 when T * E * d >= 2^30; else fused when
                               T <= 1024, E <= 256 and E * d <= 2^16; else float64 */
  MOE_ROUTER_FLOAT64 = 1,   /* every logit summed in float64 (split-K tiles) */
  MOE_ROUTER_SCREENED = 2,  /* bf16 only: MFMA logits with a proven error bound pick the
                               candidates; only candidates get the float64 sum */
  MOE_ROUTER_FUSED = 3      /* small batches only (T <= 1024, E <= 256, E * d <= 2^19; other
                               shapes: MOE_ERR_UNSUPPORTED): every logit summed in float64
                               by one workgroup per token, offsets and selection in the
                               same launch */
} moe_router;

/* Budget each token executes, from its requested k_t (validated first: a
 * k_t outside [0, k_max] is flagged and runs as 0 under every policy).
 * EXACT runs k_t.  The other two are the over-serving comparators of
 * MoE-Prism: BATCH_MAX runs the batch-level maximum budget for every token
 * with a valid budget (§III-C1: a dispatch that mixes budgets uses the
 * largest one so that every request gets at least its own); ROUND_UP runs
 * N * ceil(k_t / N), N = k_granule (§V-D1: a whole-expert layout with N
 * sub-experts per expert can only execute multiples of N). */
typedef enum {
  MOE_K_EXACT = 0,
  MOE_K_BATCH_MAX = 1,
  MOE_K_ROUND_UP = 2
} moe_k_policy;

/* Workspace owners, for moe_workspace_size. */
typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_FFN = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_FORWARD = 4,
  MOE_OP_FOLD = 5,
  MOE_OP_PATH = 6   /* moe_path_route and moe_path_sources */
} moe_op;

/* Expert-folding selectors, for moe_fold. */
typedef enum {
  MOE_FOLD_TOKEN = 0,  /* per token: keep at most `budget` routes (prefill) */
  MOE_FOLD_POOL = 1    /* per batch: keep a pool of `budget` experts (decode) */
} moe_fold_mode;

/* Storage order of the expert weight matrices.  Both describe the same
 * [N][K] matrices (N output rows, K inputs); only the byte order differs.
 * BLOCKED64 cuts each matrix into (N/64) x (K/EB) blocks of 64 rows x 128
 * bytes (EB = 128 / sizeof(ELT): 64 bf16 or 32 float), block (nb, kb) at
 * element offset (nb * (K/EB) + kb) * 64 * EB, rows of the block one after
 * another: element (n, k) sits at
 *     ((n / 64) * (K / EB) + k / EB) * 64 * EB + (n % 64) * EB + k % EB,
 * and the matrices of a stack follow each other as in the row-major layout
 * (matrix e at e * N * K).  One 64-element step of K over a 64-row tile is
 * then 8 KB of contiguous memory instead of 64 lines one matrix row apart, which
 * is how the FFN kernels read it (moe_pack_weights converts). */
typedef enum {
  MOE_W_ROWMAJOR = 0,
  MOE_W_BLOCKED64 = 1
} moe_weight_layout;

/* Device status bits written by moe_route / moe_forward. */
#define MOE_DEV_BAD_K 1  /* some k_t was outside [0, k_max]; it was run as k_t = 0 */

/*
 * Layer descriptor.  Supported ranges:
 *   0 <= T, T * k_max < 2^31
 *   d, I: multiples of 128, 128 <= d, I <= 65536
 *   1 <= E <= 1024, 1 <= k_max <= E
 *   I_shared: 0 (no shared expert) or a multiple of 128 up to 65536
 *   dtype: MOE_F32 or MOE_BF16; path: a moe_path value; router: a moe_router
 *   value (MOE_ROUTER_SCREENED needs bf16)
 *   routed_scale: finite (1.0 for the plain renormalised softmax)
 *   k_policy: a moe_k_policy value; k_granule: N >= 1 for MOE_K_ROUND_UP,
 *   with k_max a multiple of N (ignored by the other policies)
 *   weight_layout: a moe_weight_layout value (0, row-major, when the field is
 *   zero-initialised)
 */
typedef struct moe_desc {
  int32_t T;            /* tokens in the batch */
  int32_t d;            /* hidden size */
  int32_t E;            /* routed experts */
  int32_t I;            /* intermediate size of one routed expert */
  int32_t k_max;        /* upper bound on every k_t */
  int32_t I_shared;     /* intermediate size of the always-on shared expert, 0 = none */
  int32_t dtype;        /* moe_dtype */
  int32_t path;         /* moe_path */
  int32_t router;       /* moe_router */
  float routed_scale;   /* factor applied to the renormalised routing weights */
  int32_t k_policy;     /* moe_k_policy: budget each token executes */
  int32_t k_granule;    /* N of MOE_K_ROUND_UP */
  int32_t weight_layout; /* moe_weight_layout of every expert weight argument */
} moe_desc;

/* Stream handle: a hipStream_t, or NULL for the null stream. */
typedef void* moe_stream_t;

/*
 * Bytes of scratch that entry point `op` needs for `desc` (a multiple of
 * 256; workspaces must be 256-byte aligned).  MOE_OP_FORWARD covers every
 * other op as well.  A size of 0 means the op takes no workspace (ws may be
 * NULL).  Host only.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED.
 */
moe_status moe_workspace_size(const moe_desc* desc, int32_t op, size_t* bytes);

/*
 * Not a step of the method (the pages fix no storage order for the expert
 * weights): a load-time conversion of this library.
 * Re-lay G row-major [N][K] matrices (contiguous, matrix g at g * N * K) into
 * the MOE_W_BLOCKED64 order; a weight stack is converted once, when it is
 * loaded, and then passed with desc->weight_layout = MOE_W_BLOCKED64.  A pure
 * permutation of elements (bit-exact).
 *   dtype   MOE_F32 or MOE_BF16 (sets EB above)
 *   G       matrices, >= 0 (0: nothing is launched)
 *   N, K    rows and columns of each: N a multiple of 64, K a multiple of
 *           128 / sizeof(ELT), both >= 1, G * N * K < 2^40
 *   src     ELT [G][N][K] row-major (16-byte aligned)
 *   dst     ELT, G * N * K elements out (16-byte aligned); must not overlap src
 * Errors: MOE_ERR_NULL, MOE_ERR_UNSUPPORTED (dtype), MOE_ERR_SHAPE (sizes, or
 * src and dst overlap), MOE_ERR_ALIGN, MOE_ERR_LAUNCH.
 */
moe_status moe_pack_weights(int32_t dtype, int32_t G, int32_t N, int32_t K, const void* src, void* dst,
                            moe_stream_t stream);

/*
 * The FFN path `desc->path` resolves to, for the routed experts and for the
 * shared expert (MOE_PATH_STREAM or MOE_PATH_GEMM).  AUTO picks the grouped
 * GEMM for bf16 when T * k_max >= 64 * E (routed) or T >= 256 (shared), i.e.
 * from the shape alone; fp32 always streams.  Host only.
 * Errors: as moe_workspace_size; MOE_ERR_UNSUPPORTED for MOE_PATH_GEMM in fp32.
 */
moe_status moe_resolve_path(const moe_desc* desc, int32_t* routed_path, int32_t* shared_path);

/*
 * Router and per-token top-k (MoE-Prism §III-B2, normalised and scaled router
 * weights of the selected experts ordered by router probability; §III-C1,
 * per-request budget).
 *   x           ELT [T][d]
 *   w_router    ELT [E][d]
 *   router_bias float [E], or NULL for none (added to the logits before selection)
 *   k           int32 [T], per-token budgets
 *   tok_off     int32 [T+1] out: exclusive prefix sum of the executed budgets (the
 *               validated k_t under desc->k_policy); tok_off[T] = A
 *   topk_ids    int32 [T*k_max] out: ids of token t at tok_off[t] .. tok_off[t+1]-1,
 *               best first
 *   topk_w      float [T*k_max] out: w_j = routed_scale * exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
 *   dev_status  int32 [1] out, or NULL: MOE_DEV_BAD_K if some k_t < 0 or > k_max
 *               (such a token is routed to no expert); 0 otherwise
 *   ws          scratch of moe_workspace_size(MOE_OP_ROUTE) bytes
 */
moe_status moe_route(const moe_desc* desc, const void* x, const void* w_router,
                     const float* router_bias, const int32_t* k, int32_t* tok_off,
                     int32_t* topk_ids, float* topk_w, int32_t* dev_status,
                     void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Dispatch metadata: a stable counting sort of the A assignments by
 * (expert ascending, token ascending).  Deterministic and bit-exact.
 *   tok_off, topk_ids  from moe_route
 *   expert_counts int32 [E] out: assignments per expert
 *   expert_off    int32 [E+1] out: exclusive scan of expert_counts
 *   perm_tok      int32 [T*k_max] out: token of sorted row p
 *   perm_src      int32 [T*k_max] out: assignment index tok_off[t]+j of sorted row p
 *   inv_perm      int32 [T*k_max] out: sorted row of assignment a; -1 for an
 *                 assignment whose expert id is outside [0, E) (never
 *                 produced by moe_route: such an entry gets no row, is not
 *                 counted, and moe_combine skips it)
 *   n_active      int32 [1] out: experts with at least one assignment
 *                 (the activated experts whose weights a batch loads; METRO
 *                 reading notes, arXiv 2512.09277, Q1)
 *   ws            scratch of moe_workspace_size(MOE_OP_PERMUTE) bytes
 */
moe_status moe_permute(const moe_desc* desc, const int32_t* tok_off, const int32_t* topk_ids,
                       int32_t* expert_counts, int32_t* expert_off, int32_t* perm_tok,
                       int32_t* perm_src, int32_t* inv_perm, int32_t* n_active,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Grouped SwiGLU expert FFN over the permuted rows (MoE-Prism §III-B1,
 * Eq. (1)): for expert e and sorted row p in [expert_off[e], expert_off[e+1]),
 *   H[p] = SiLU(x[perm_tok[p]] . w_gate[e]^T) * (x[perm_tok[p]] . w_up[e]^T)
 *   y_perm[p] = H[p] . w_down[e]^T
 * with float32 accumulation; H is kept in ELT.  With a shared expert
 * (I_shared > 0) the same FFN runs on every token with ws_* into y_shared.
 *   y_perm    ELT [T*k_max][d] out (rows >= A untouched)
 *   y_shared  ELT [T][d] out; ignored (may be NULL) when I_shared == 0
 *   ws        scratch of moe_workspace_size(MOE_OP_FFN) bytes (holds H)
 * The per-expert row counts are read on the device.
 */
moe_status moe_ffn(const moe_desc* desc, const void* x, const void* w_gate, const void* w_up,
                   const void* w_down, const void* ws_gate, const void* ws_up,
                   const void* ws_down, const int32_t* expert_off, const int32_t* perm_tok,
                   void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                   moe_stream_t stream);

/*
 * The routed part of moe_ffn as three calls, so that a caller can place or
 * time the two FFN halves separately (one kernel launch each):
 *   moe_ffn_plan:   writes the row-block work table of the FFN kernels into
 *                   `ws` from expert_off (one one-workgroup kernel).  Each
 *                   expert's rows are cut into fixed-size blocks and listed;
 *                   the list's length bound depends on the shape only, so the
 *                   FFN launch grids do too.  Must precede moe_ffn_gateup /
 *                   moe_ffn_down on the same `ws` and stream, and be repeated
 *                   whenever expert_off changes.
 *   moe_ffn_gateup: h ELT [T*k_max][I] out, H of the rows above.
 *   moe_ffn_down:   y_perm ELT [T*k_max][d] out from h.
 * `ws`: scratch of moe_workspace_size(MOE_OP_FFN) bytes (may be shared with
 * moe_ffn's; h must not alias it).  Errors: as moe_ffn.
 */
moe_status moe_ffn_plan(const moe_desc* desc, const int32_t* expert_off, void* ws, size_t ws_bytes,
                        moe_stream_t stream);
moe_status moe_ffn_gateup(const moe_desc* desc, const void* x, const void* w_gate,
                          const void* w_up, const int32_t* expert_off, const int32_t* perm_tok,
                          void* h, void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status moe_ffn_down(const moe_desc* desc, const void* h, const void* w_down,
                        const int32_t* expert_off, void* y_perm, void* ws, size_t ws_bytes,
                        moe_stream_t stream);

/*
 * Expert folding of the routing metadata (ExFold summary, arXiv 2608.24938:
 * Unified Expert Folding; Phase-Specific Selection and Unified Folding;
 * Phase-Specific Routing and Folding).  The routes of moe_route are cut to a
 * budget, and every dropped route is folded into a kept one: its target is the
 * kept expert of smallest projection loss L[source][target], and the dropped
 * weight times the scalar projector S[source][target] is added to the
 * target's weight.  Expert weights and the router are untouched; the folded
 * routes feed moe_permute / moe_ffn / moe_combine like moe_route's.
 *   mode = MOE_FOLD_TOKEN: a token with more than `budget` routes keeps the
 *     `budget` largest by topk_w * H[e] (ties: earlier route), in their
 *     original order; ties in L go to the earlier kept route.
 *   mode = MOE_FOLD_POOL: the pool is the `budget` activated experts with the
 *     largest H[e] * (sum of the weights routed to e, float64, in token
 *     order), ties to the lower index; a route outside the pool goes to the
 *     pool expert of smallest L (ties: lower index); a token's routes that
 *     land on one expert are merged at the first one's place, weights added
 *     in route order.  Needs expert_off / perm_src of moe_permute on the
 *     input routes (the weights are summed in that row order).
 *   S, L         float [E][E] (row: dropped source, column: target)
 *   H            float [E], expert output magnitudes (>= 0)
 *   tok_off, topk_ids, topk_w   input routes (moe_route's CSR)
 *   expert_off, perm_src        MOE_FOLD_POOL only (else may be NULL)
 *   tok_off_out  int32 [T+1] out; ids_out int32 [T*k_max] out; w_out float [T*k_max] out
 *   pool_out     int32 [E] out (1: in the pool), or NULL; MOE_FOLD_POOL only
 *   ws           scratch of moe_workspace_size(MOE_OP_FOLD) bytes
 * A route whose expert id is outside [0, E) is dropped without a target.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (budget < 1, or k_max > 64),
 * MOE_ERR_UNSUPPORTED (mode), MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 */
moe_status moe_fold(const moe_desc* desc, int32_t mode, int32_t budget, const float* S, const float* L,
                    const float* H, const int32_t* tok_off, const int32_t* topk_ids, const float* topk_w,
                    const int32_t* expert_off, const int32_t* perm_src, int32_t* tok_off_out,
                    int32_t* ids_out, float* w_out, int32_t* pool_out, void* ws, size_t ws_bytes,
                    moe_stream_t stream);

/*
 * Training-free proxy gating of a split layer (MoE-Prism, arXiv 2510.19366,
 * §III-B2, Training-Free Proxy Gating).  `desc` describes the split layer: E
 * sub-experts of width I, sub-expert n of whole expert e at index N*e + n
 * (E a multiple of N), budgets k_t counted in sub-experts, k_max <= m*N and
 * m*N <= 64.  The whole-expert router picks m experts per token (moe_route on
 * a descriptor with E/N experts, k_max = m and every k_t = m); the N
 * sub-experts of the j-th pick get proxy scores s_n = mean over the r gate
 * neurons c of |SiLU(x . w_gate[c]) * (x . w_up[c])|; the kappa_j best run
 * (ties: lower n), each with the pick's routing weight (no second softmax).
 *
 * The proxy weight set of whole expert e has Ip = N*r rounded up to a multiple
 * of 128 rows: row n*r + i is gate neuron i of sub-expert N*e + n, the rows
 * from N*r on are zero.
 *
 * Precision (the pages fix none; the contract is the router's): g = x .
 * w_gate[c] and u = x . w_up[c] are exact products summed in float64 and
 * rounded once to float32 each; |SiLU(g) u| = |g / (1 + exp(-g)) * u| and
 * the mean over the r neurons (summed in neuron order, then divided by r) are
 * float64, and the picks are decided on those float64 scores.
 *
 * moe_proxy_pack: gathers the gate-neuron rows once per layer.
 *   gate_idx  int32 [E][r]: neurons (rows of the sub-expert's w_gate / w_up);
 *             one outside [0, I) packs as a zero row (its activation is 0)
 *   w_gate, w_up  ELT [E][I][d];  wp_gate, wp_up  ELT [E/N][Ip][d] out
 * moe_proxy_route: routes of the split layer from the proxy scores.
 *   k       int32 [T] sub-expert budgets
 *   kappa   int32 [k_max+1][m]: kappa vector of each budget k (0 <= kappa_j
 *           <= N, sum_j kappa_j = k); a token with budget k_t runs k_t routes
 *   base_tok_off, base_ids, base_w   the whole-expert routes (moe_route on
 *           a descriptor with E/N experts, k_max = m, every k_t = m)
 *   base_expert_off, base_perm_tok, base_perm_src   moe_permute's expert_off,
 *           perm_tok and perm_src on those routes (the scores are taken per
 *           block of up to 64 permuted rows of one whole expert)
 *   x       ELT [T][d] the tokens' hidden states
 *   wp_gate, wp_up  ELT [E/N][Ip][d]: moe_proxy_pack's output (desc's
 *           weight layout)
 *   tok_off int32 [T+1], topk_ids int32 [T*k_max], topk_w float [T*k_max] out
 *           (CSR like moe_route's; within a pick, chosen sub-experts by
 *           score; a whole-expert pick outside [0, E/N) fills its kappa_j
 *           slots with id -1 and weight 0, which moe_permute and moe_combine
 *           skip)
 *   dev_status int32 [1] out or NULL: MOE_DEV_BAD_K for a k_t outside
 *           [0, k_max] or whose kappa row has an entry outside [0, N] or does
 *           not sum to k_t (such a token runs nothing)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (N, r, m out of range), MOE_ERR_ALIGN
 * (the weights, or x), MOE_ERR_LAUNCH.
 */
/*
 * moe_proxy_kappa_balanced (host only, no device call): the kappa table of
 * moe_proxy_route with each budget k split as evenly as possible over the m
 * picks, the remainder going to the earlier picks (higher router
 * probability): kappa[k][j] = k / m + (j < k % m).
 *   kappa  int32 [k_max+1][m] host memory, out.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (m < 1, N < 1, k_max < 0 or k_max > m*N).
 */
moe_status moe_proxy_kappa_balanced(int32_t k_max, int32_t m, int32_t N, int32_t* kappa);
moe_status moe_proxy_pack(const moe_desc* desc, int32_t N, int32_t r, const int32_t* gate_idx,
                          const void* w_gate, const void* w_up, void* wp_gate, void* wp_up,
                          moe_stream_t stream);
moe_status moe_proxy_route(const moe_desc* desc, int32_t N, int32_t r, int32_t m, const int32_t* k,
                           const int32_t* kappa, const int32_t* base_tok_off, const int32_t* base_ids,
                           const float* base_w, const int32_t* base_expert_off, const int32_t* base_perm_tok,
                           const int32_t* base_perm_src, const void* x, const void* wp_gate, const void* wp_up,
                           int32_t* tok_off, int32_t* topk_ids, float* topk_w, int32_t* dev_status,
                           moe_stream_t stream);

/*
 * Compositional paths (PCoMoE, arXiv 2609.01024).  Expert e splits at its
 * expansion/projection boundary into U_e(h) = SiLU(h . w_gate[e]) * (h .
 * w_up[e]) and D_e(z) = z . w_down[e]; a path (i, j) is D_j(U_i(h)), and the
 * diagonal (e, e) is the vanilla expert.  A fixed list of active paths (the
 * pruned mask, materialised offline) holds the candidates; a token runs its
 * k_t best paths (k_t counted in paths, k_max <= 64 and <= the list length),
 * and each distinct source's expansion runs once per token (source-grouped
 * reuse):  out = sum_i sum_{j in T_i} beta_ij D_j(U_i(h)).
 *
 * moe_path_table_bytes / moe_path_table: validate the active list on the host
 * and upload it (once per layer).  src, tgt int32 [P] and bias float [P] are
 * host arrays: 1 <= P <= 1024, entries in [0, E), (src, tgt) strictly
 * increasing, biases finite.  `table` is device memory of
 * moe_path_table_bytes(P) bytes (16-byte aligned); the call returns once the
 * copy is complete.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (any rule above),
 * MOE_ERR_ALIGN, MOE_ERR_LAUNCH.
 *
 * moe_path_route: per token, the router logits g = x . w_router^T (+ bias) and,
 * when w_tgt is not NULL, the target prior t = x . w_tgt^T, both under
 * moe_route's contract (float64 accumulation, one rounding to float32); path
 * scores s_p = fp32((g[src_p] + bias_p) + lambda * t[tgt_p]) in float64
 * (compatibility-aware path gating, Fig. 7); the k_t best paths (score
 * descending, equal scores in list order) with weights beta = routed_scale *
 * softmax over the selected scores (the renormalised softmax, so the
 * diagonal-only list with zero biases reproduces moe_route exactly).
 *   w_tgt     ELT [E][d] or NULL; lambda ignored when NULL
 *   k         int32 [T]; budgets follow desc.k_policy as in moe_route
 *   tok_off   int32 [T+1] out; path_src, path_tgt int32 [T*k_max] out;
 *   path_w    float [T*k_max] out; dev_status as in moe_route
 *   ws        scratch of moe_workspace_size(MOE_OP_PATH) bytes
 * moe_path_sources: the source groups (Fig. 8): per token its distinct
 * sources in ascending order (src_tok_off int32 [T+1], src_ids int32
 * [T*k_max]), the source route of every path (path_src_route int32
 * [T*k_max]), and unit_off int32 [T*k_max+1] = min(a, A): the offsets of the
 * paths taken one per row, for moe_permute of path_tgt under a descriptor of
 * T*k_max tokens with k_max = 1 (a token may reach one target through two
 * sources).  ws: as moe_path_route's.
 * moe_path_rows: row_map[q] = src_inv_perm[path_src_route[perm_path[q]]] for
 * q < A = tok_off[T]: the expansion row (of moe_ffn_gateup over the source
 * routes) that target-ordered path row q reads; perm_path is the perm_tok of
 * the one-per-row permutation above (its "tokens" are the paths).
 * moe_ffn_down_rows: moe_ffn_down where permuted row p reads h row
 * row_map[p] (int32 [T*k_max]).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (k_max > 64 or > P, P out of range,
 * lambda not finite), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 */
moe_status moe_path_table_bytes(int32_t P, size_t* bytes);
moe_status moe_path_table(int32_t E, int32_t P, const int32_t* src, const int32_t* tgt, const float* bias,
                          void* table, size_t table_bytes, moe_stream_t stream);
moe_status moe_path_route(const moe_desc* desc, const void* x, const void* w_router, const float* router_bias,
                          const void* w_tgt, float lambda, const void* table, int32_t P, const int32_t* k,
                          int32_t* tok_off, int32_t* path_src, int32_t* path_tgt, float* path_w,
                          int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status moe_path_sources(const moe_desc* desc, const int32_t* tok_off, const int32_t* path_src,
                            int32_t* src_tok_off, int32_t* src_ids, int32_t* path_src_route, int32_t* unit_off,
                            void* ws, size_t ws_bytes, moe_stream_t stream);
moe_status moe_path_rows(const moe_desc* desc, const int32_t* tok_off, const int32_t* perm_path,
                         const int32_t* path_src_route, const int32_t* src_inv_perm, int32_t* row_map,
                         moe_stream_t stream);
moe_status moe_ffn_down_rows(const moe_desc* desc, const void* h, const int32_t* row_map, const void* w_down,
                             const int32_t* expert_off, void* y_perm, void* ws, size_t ws_bytes,
                             moe_stream_t stream);

/*
 * Weighted combine back to token order: the routed output of a token is the
 * sum of its selected experts' FFN outputs, each scaled by its normalised
 * router weight (MoE-Prism, arXiv 2510.19366, §III-B2, training-free proxy
 * gating: the routed output is the w_j-weighted sum of the executed experts'
 * FFNs; PCoMoE, arXiv 2609.01024, Compositional Path Routing: the vanilla layer
 * is the weighted expert summation), plus the always-on shared expert with
 * weight 1 (§II-B: shared experts are outside the routed budget):
 *   out[t] = sum_{j < k_t} topk_w[tok_off[t]+j] * y_perm[inv_perm[tok_off[t]+j]]
 *            (+ y_shared[t] when y_shared != NULL)
 * summed in float32 in ascending j, rounded once to ELT.  A token with
 * k_t = 0 gets y_shared[t] (or 0).  An assignment whose inv_perm entry is
 * negative (moe_permute writes -1 for an expert id outside [0, E)) adds
 * nothing.
 *   y_perm    ELT [T*k_max][d] in: expert outputs in permuted row order
 *   y_shared  ELT [T][d] in, or NULL
 *   tok_off, topk_w, inv_perm: as written by moe_route / moe_permute
 *   out       ELT [T][d] out
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN (y_perm, y_shared, out), MOE_ERR_LAUNCH.
 */
moe_status moe_combine(const moe_desc* desc, const void* y_perm, const void* y_shared,
                       const int32_t* tok_off, const float* topk_w, const int32_t* inv_perm,
                       void* out, moe_stream_t stream);

/*
 * The whole layer: route, permute, FFN (+ shared expert) and combine.  Per
 * token t with budget k_t (MoE-Prism §III-C1: the request carries its own
 * routing budget, counted in routed experts, §II-B), the output is the
 * renormalised-softmax-weighted sum over the k_t highest-logit experts of the
 * SwiGLU expert FFN (§III-B1, Eq. (1): A = SiLU(X W_gate) * (X W_up), output
 * A W_down), plus the shared expert's output; the steps are those of
 * moe_route, moe_permute, moe_ffn and moe_combine above.
 *   x, w_router, router_bias, k: as in moe_route
 *   w_gate, w_up, w_down, ws_gate, ws_up, ws_down: as in moe_ffn
 *   out        ELT [T][d] out
 *   stats      int32 [E+2] out, or NULL: expert_counts[E], n_active, A
 *   dev_status int32 [1] out, or NULL: as in moe_route
 *   ws         scratch of moe_workspace_size(MOE_OP_FORWARD) bytes; it also
 *              holds the routing and permutation arrays of the call
 */
moe_status moe_forward(const moe_desc* desc, const void* x, const void* w_router,
                       const float* router_bias, const int32_t* k, const void* w_gate,
                       const void* w_up, const void* w_down, const void* ws_gate,
                       const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                       int32_t* dev_status, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Streaming-read probe (measurement only, not a step of the layer): reads
 * `bytes` bytes of device memory at src once with 16-byte loads, carrying
 * the non-temporal hint when `nontemporal` is non-zero, as a plain kernel
 * that does nothing else; timing it gives the HBM read rate this part
 * reaches, the practical ceiling of a weight stream.
 *   src   device, 16-byte aligned; bytes rounded down to a multiple of 16
 *   sink  device int32 [1]; written only in the practically impossible case
 *         that the folded data equal a fixed constant (it keeps the loads)
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_LAUNCH.
 */
moe_status moe_probe_read(const void* src, size_t bytes, int32_t nontemporal, int32_t* sink,
                          moe_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP-graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_forward with its scratch in a library-held device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace.  Same
 * arguments, kernels and results as moe_forward, minus ws / ws_bytes; the
 * caller still passes every input and output.  Calls nothing that allocates.
 *   - The array is a static device variable: each GPU the library runs on
 *     holds its own copy until the process ends.  Its address is looked up
 *     on the first call on a device (with that device current).
 *   - Layers whose forward needs more scratch than the array holds are
 *     rejected with MOE_ERR_SCRATCH before anything is launched (the decode
 *     shapes fit: about 30 MiB at most; large prefill batches do not).
 *   - Every call on a GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (two streams, two host threads) race and give wrong
 *     results.  Nothing in the array needs clearing between calls (every
 *     region is written before it is read).
 * Errors: those of moe_forward (other than MOE_ERR_WORKSPACE), MOE_ERR_SCRATCH.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                               const float* router_bias, const int32_t* k, const void* w_gate,
                               const void* w_up, const void* w_down, const void* ws_gate,
                               const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                               int32_t* dev_status, moe_stream_t stream);

/* Static description of a status code.  Never NULL. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
