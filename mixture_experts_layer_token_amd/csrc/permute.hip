// Dispatch metadata of the grouped expert FFN: per-expert histogram, exclusive
// scan and a stable counting-sort permutation of the assignments by
// (expert, token).  Integer work only; bit-exact and run-to-run deterministic
// (LDS atomics are used only for order-free OR).
//
// Tokens are cut into blocks of 256.  In each block every expert owns a
// 256-bit mask of the tokens that selected it (a token selects an expert at
// most once).  The rank of (t, e) inside its block is the popcount of e's mask
// below t, so the global row is
//   expert_off[e] + block_base[blk][e] + popcount(mask_e & below(t)).
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int MASK_WORDS = PERM_BLOCK / 32;

// ---------------------------------------------------------------------------
// Row-block table of the grouped FFN (declared in launch.h).
int row_block_bound(int A_cap, int G, int RB) { return A_cap / RB + min(G, A_cap); }

// Group g's entries (rows [r0, r0 + n)) from table index `start` on.
__device__ __forceinline__ void put_row_blocks(int4* __restrict__ blocks, int g, int r0, int n, int RB, int start,
                                               int bound) {
  for (int b = 0, i = start; b * RB < n && i < bound; ++b, ++i) blocks[i] = make_int4(g, r0 + b * RB, min(RB, n - b * RB), 0);
}
// Sentinels after the `count` real entries and the count itself at `bound`.
__device__ __forceinline__ void close_row_blocks(int4* __restrict__ blocks, int count, int bound, int tid,
                                                 int nthreads) {
  count = min(count, bound);
  for (int i = count + tid; i < bound; i += nthreads) blocks[i] = make_int4(-1, 0, 0, 0);
  if (tid == 0) blocks[bound] = make_int4(count, 0, 0, 0);
}

// Inclusive scan of one value per thread over a workgroup of NT threads
// (`sc` provides the NT / 64 wave totals).
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int32_t* sc) {
  return block_scan_incl<NT>(v, sc);
}

__global__ __launch_bounds__(1024) void row_blocks_kernel(const int32_t* __restrict__ grp_off, int G, int RB,
                                                          int bound, int4* __restrict__ blocks) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t total;
  const int g = threadIdx.x;
  int r0 = 0, n = 0;
  if (g < G) {
    r0 = grp_off[g];
    n = max(0, grp_off[g + 1] - r0);
  }
  const int nb = (n + RB - 1) / RB;
  const int incl = block_inclusive_scan<1024>(nb, sc);
  if (g == 1023) total = incl;
  __syncthreads();
  put_row_blocks(blocks, g, r0, n, RB, incl - nb, bound);
  close_row_blocks(blocks, total, bound, g, 1024);
}

hipError_t launch_row_blocks(const int32_t* grp_off, int G, int RB, int bound, int4* blocks, hipStream_t st) {
  hipLaunchKernelGGL(row_blocks_kernel, dim3(1), dim3(1024), 0, st, grp_off, G, RB, bound, blocks);
  return hipGetLastError();
}

// Calls f(a, e) for each assignment a in [a0, a1) of one token with its expert
// id e; the ids are loaded eight at a time, so that their latencies overlap
// instead of adding up (a token's k_t loads otherwise wait one after another).
template <class F>
__device__ __forceinline__ void for_token_ids(const int32_t* __restrict__ ids, int a0, int a1, F f) {
  for (int b = a0; b < a1; b += 8) {
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (b + j < a1) ? ids[b + j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (b + j < a1) f(b + j, e[j]);
  }
}

__device__ __forceinline__ void build_masks(uint32_t* masks, const int32_t* __restrict__ tok_off,
                                            const int32_t* __restrict__ ids, int T, int E) {
  const int tid = threadIdx.x;
  for (int i = tid; i < E * MASK_WORDS; i += PERM_BLOCK) masks[i] = 0u;
  __syncthreads();
  const int t = blockIdx.x * PERM_BLOCK + tid;
  if (t < T) {
    const uint32_t bit = 1u << (tid & 31);
    for_token_ids(ids, tok_off[t], tok_off[t + 1], [&](int, int e) {
      if ((unsigned)e < (unsigned)E) atomicOr(&masks[e * MASK_WORDS + (tid >> 5)], bit);
    });
  }
  __syncthreads();
}

__global__ __launch_bounds__(PERM_BLOCK) void expert_hist_kernel(const int32_t* __restrict__ tok_off,
                                                                 const int32_t* __restrict__ ids, int T, int E,
                                                                 int32_t* __restrict__ block_counts) {
  extern __shared__ uint32_t masks[];
  build_masks(masks, tok_off, ids, T, E);
  for (int e = threadIdx.x; e < E; e += PERM_BLOCK) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < MASK_WORDS; ++w) c += __popc(masks[e * MASK_WORDS + w]);
    block_counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// Many blocks (large batches): one workgroup per expert adds the expert's
// block counts and writes their exclusive prefix (block_base) and total
// (counts), so the one-workgroup scan below only scans the experts.
__global__ __launch_bounds__(256) void expert_block_scan_kernel(const int32_t* __restrict__ block_counts, int nblk,
                                                                int E, int32_t* __restrict__ block_base,
                                                                int32_t* __restrict__ counts) {
  __shared__ int32_t wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int per = (nblk + 255) / 256;
  const int b0 = min(tid * per, nblk), b1 = min(b0 + per, nblk);
  int s = 0;
#pragma unroll 16
  for (int bb = b0; bb < b1; ++bb) s += block_counts[(size_t)bb * E + e];
  const int incl = block_scan_incl<256>(s, wsum);
  int r = incl - s;
#pragma unroll 16
  for (int bb = b0; bb < b1; ++bb) {
    block_base[(size_t)bb * E + e] = r;
    r += block_counts[(size_t)bb * E + e];
  }
  if (tid == 255) counts[e] = incl;
}

// One workgroup: per-expert running sums over blocks, then the exclusive scan
// over experts.  With `presummed` the totals are already in counts and the
// block bases written (expert_block_scan_kernel).  Q = 1024 / E' threads share an expert (E' = E rounded up to a
// power of two): thread (e, q) sums a contiguous run of blocks, the runs'
// sums are scanned per expert, then every thread writes its blocks' bases.
__global__ __launch_bounds__(1024) void expert_scan_kernel(const int32_t* __restrict__ block_counts, int nblk,
                                                           int E, int Q, int32_t* __restrict__ block_base,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ expert_off,
                                                           int32_t* __restrict__ n_active,
                                                           int32_t* __restrict__ stats, int RB, int bound,
                                                           int4* __restrict__ blocks, int presummed) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t qsum[1024];
  __shared__ int32_t nact, nblocks;
  const int tid = threadIdx.x;
  const int e = tid / Q, q = tid - (tid / Q) * Q;  // Q is a power of two dividing 1024
  const int per = (nblk + Q - 1) / Q;
  const int b0 = min(q * per, nblk), b1 = min(b0 + per, nblk);
  int part = 0;
  if (presummed) {
    part = (q == 0 && e < E) ? counts[e] : 0;
  } else if (e < E) {
    // 32 loads in flight per round: with many blocks (large batches) the run
    // is hundreds of loads long
#pragma unroll 32
    for (int bb = b0; bb < b1; ++bb) part += block_counts[(size_t)bb * E + e];
  }
  qsum[tid] = part;
  if (tid == 0) nact = 0;
  __syncthreads();
  // exclusive prefix of the runs of expert e, and its total
  int before = 0, run = 0;
  for (int j = 0; j < Q; ++j) {
    const int v = qsum[e * Q + j];
    if (j < q) before += v;
    run += v;
  }
  if (e < E && !presummed) {
    int r = before;
#pragma unroll 32
    for (int bb = b0; bb < b1; ++bb) {
      block_base[(size_t)bb * E + e] = r;
      r += block_counts[(size_t)bb * E + e];
    }
  }
  // one thread per expert continues with the expert scan
  const bool lead = q == 0 && e < E;
  if (lead) {
    counts[e] = run;
    if (stats) stats[e] = run;
    if (run > 0) atomicAdd(&nact, 1);
  }
  __syncthreads();
  const int ev = (q == 0 && e < E) ? run : 0;  // one contribution per expert, in expert order
  // scan over experts in the order of e (thread tid = e * Q holds expert e)
  const int incl = block_scan_incl<1024>(ev, sc);
  const int first = incl - ev;
  if (lead) expert_off[e] = first;
  if (tid == 1023) {
    expert_off[E] = incl;
    n_active[0] = nact;
    if (stats) {
      stats[E] = nact;
      stats[E + 1] = incl;
    }
  }
  if (blocks) {
    __syncthreads();
    const int nb = lead ? (run + RB - 1) / RB : 0;
    const int incl = block_inclusive_scan<1024>(nb, sc);
    if (tid == 1023) nblocks = incl;
    __syncthreads();
    if (lead) put_row_blocks(blocks, e, first, run, RB, incl - nb, bound);
    close_row_blocks(blocks, nblocks, bound, tid, 1024);
  }
}

// Scatter: SPLIT workgroups per 256-token block, each placing the assignments
// of 256 / SPLIT of its tokens.  Every workgroup rebuilds the block's masks and
// the per-word popcount prefixes, so a rank is two LDS reads.
constexpr int SCATTER_SPLIT = 4;

__global__ __launch_bounds__(PERM_BLOCK) void expert_scatter_kernel(
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ ids, int T, int E, int k_max,
    const int32_t* __restrict__ block_base, const int32_t* __restrict__ expert_off,
    int32_t* __restrict__ perm_tok, int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm) {
  extern __shared__ uint32_t masks[];
  int32_t* const wpre = reinterpret_cast<int32_t*>(masks + E * MASK_WORDS);  // [E][MASK_WORDS]
  const int blk = blockIdx.x / SCATTER_SPLIT, part = blockIdx.x - blk * SCATTER_SPLIT;
  const int tid = threadIdx.x;
  // masks of the whole block
  for (int i = tid; i < E * MASK_WORDS; i += PERM_BLOCK) masks[i] = 0u;
  __syncthreads();
  {
    const int t = blk * PERM_BLOCK + tid;
    if (t < T) {
      const uint32_t bit = 1u << (tid & 31);
      for_token_ids(ids, tok_off[t], tok_off[t + 1], [&](int, int e) {
        if ((unsigned)e < (unsigned)E) atomicOr(&masks[e * MASK_WORDS + (tid >> 5)], bit);
      });
    }
  }
  __syncthreads();
  // global base of (block, expert) plus the popcounts of the words before w
  for (int e = tid; e < E; e += PERM_BLOCK) {
    int r = expert_off[e] + block_base[(size_t)blk * E + e];
#pragma unroll
    for (int w = 0; w < MASK_WORDS; ++w) {
      wpre[e * MASK_WORDS + w] = r;
      r += __popc(masks[e * MASK_WORDS + w]);
    }
  }
  __syncthreads();
  // this workgroup's tokens: one thread per (token, assignment slot j < 64)
  constexpr int TPW = PERM_BLOCK / SCATTER_SPLIT;  // tokens per workgroup
  const int tl0 = part * TPW;
  const int slots = min(k_max, 64);
  for (int i = tid; i < TPW * slots; i += PERM_BLOCK) {
    const int tl = tl0 + (i & (TPW - 1)), j = i / TPW;  // token within the block, its j-th assignment
    const int t = blk * PERM_BLOCK + tl;
    if (t >= T) continue;
    const int a0 = tok_off[t], a1 = tok_off[t + 1];
    if (a0 + j >= a1) continue;
    const int a = a0 + j;
    const int e = ids[a];
    if ((unsigned)e >= (unsigned)E) {  // not produced by moe_route: no row, and the combine skips it
      inv_perm[a] = -1;
      continue;
    }
    const int wi = tl >> 5;
    const int pos = wpre[e * MASK_WORDS + wi] + __popc(masks[e * MASK_WORDS + wi] & ((1u << (tl & 31)) - 1u));
    perm_tok[pos] = t;
    perm_src[pos] = a;
    inv_perm[a] = pos;
  }
  // assignment slots past 64 (k_t > 64): the remaining ones, thread per token
  for (int tl = tl0 + tid; tl < tl0 + TPW; tl += PERM_BLOCK) {
    const int t = blk * PERM_BLOCK + tl;
    if (t >= T) continue;
    const int a0 = tok_off[t], a1 = tok_off[t + 1];
    const int wi = tl >> 5;
    const uint32_t below = (1u << (tl & 31)) - 1u;
    for (int a = a0 + 64; a < a1; ++a) {
      const int e = ids[a];
      if ((unsigned)e >= (unsigned)E) {
        inv_perm[a] = -1;
        continue;
      }
      const int pos = wpre[e * MASK_WORDS + wi] + __popc(masks[e * MASK_WORDS + wi] & below);
      perm_tok[pos] = t;
      perm_src[pos] = a;
      inv_perm[a] = pos;
    }
  }
}

// Whole permutation in one workgroup when all tokens fit in one block
// (T <= 256, the decode batches): masks, counts, scan over experts and
// scatter without leaving LDS.
__global__ __launch_bounds__(PERM_BLOCK) void permute_one_block_kernel(
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ ids, int T, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ expert_off, int32_t* __restrict__ perm_tok, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ n_active, int32_t* __restrict__ stats, int RB, int bound,
    int4* __restrict__ blocks) {
  extern __shared__ uint32_t masks[];
  int32_t* eoff = reinterpret_cast<int32_t*>(masks + E * MASK_WORDS);  // [E + 1]
  __shared__ int32_t part[PERM_BLOCK];
  __shared__ int32_t nact, nblocks;
  build_masks(masks, tok_off, ids, T, E);
  const int tid = threadIdx.x;
  const int per = (E + PERM_BLOCK - 1) / PERM_BLOCK;
  const int beg = min(tid * per, E), end = min(beg + per, E);
  int s = 0, act = 0;
  for (int e = beg; e < end; ++e) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < MASK_WORDS; ++w) c += __popc(masks[e * MASK_WORDS + w]);
    eoff[e] = c;
    s += c;
    act += c > 0;
  }
  if (tid == 0) nact = 0;
  __syncthreads();
  if (act) atomicAdd(&nact, act);
  const int incl_s = block_scan_incl<PERM_BLOCK>(s, part);
  int run = incl_s - s;
  for (int e = beg; e < end; ++e) {
    const int c = eoff[e];
    counts[e] = c;
    if (stats) stats[e] = c;
    eoff[e] = run;
    expert_off[e] = run;
    run += c;
  }
  if (tid == PERM_BLOCK - 1) {
    eoff[E] = incl_s;
    expert_off[E] = incl_s;
    n_active[0] = nact;
    if (stats) {
      stats[E] = nact;
      stats[E + 1] = incl_s;
    }
  }
  __syncthreads();
  if (blocks) {
    // row-block table: this thread's experts, after the blocks of lower threads
    int nb = 0;
    for (int e = beg; e < end; ++e) nb += (eoff[e + 1] - eoff[e] + RB - 1) / RB;
    const int incl = block_inclusive_scan<PERM_BLOCK>(nb, part);
    if (tid == PERM_BLOCK - 1) nblocks = incl;
    __syncthreads();
    int start = incl - nb;
    for (int e = beg; e < end; ++e) {
      const int c = eoff[e + 1] - eoff[e];
      put_row_blocks(blocks, e, eoff[e], c, RB, start, bound);
      start += (c + RB - 1) / RB;
    }
    close_row_blocks(blocks, nblocks, bound, tid, PERM_BLOCK);
  }
  if (tid >= T) return;
  const int wi = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for_token_ids(ids, tok_off[tid], tok_off[tid + 1], [&](int a, int e) {
    if ((unsigned)e >= (unsigned)E) {  // not produced by moe_route: no row, and the combine skips it
      inv_perm[a] = -1;
      return;
    }
    const uint32_t* m = masks + e * MASK_WORDS;
    int rank = __popc(m[wi] & below);
    for (int w = 0; w < wi; ++w) rank += __popc(m[w]);
    const int pos = eoff[e] + rank;
    perm_tok[pos] = tid;
    perm_src[pos] = a;
    inv_perm[a] = pos;
  });
}

hipError_t launch_permute(const int32_t* tok_off, const int32_t* ids, int T, int E, int k_max, int32_t* block_counts,
                          int32_t* block_base, int32_t* counts, int32_t* expert_off, int32_t* perm_tok,
                          int32_t* perm_src, int32_t* inv_perm, int32_t* n_active, int32_t* stats, int RB,
                          int bound, int4* blocks, hipStream_t st) {
  const int nblk = (T + PERM_BLOCK - 1) / PERM_BLOCK;
  const size_t lds = (size_t)E * MASK_WORDS * sizeof(uint32_t);
  if (nblk == 1) {
    hipLaunchKernelGGL(permute_one_block_kernel, dim3(1), dim3(PERM_BLOCK), lds + (E + 1) * sizeof(int32_t), st,
                       tok_off, ids, T, E, counts, expert_off, perm_tok, perm_src, inv_perm, n_active, stats, RB,
                       bound, blocks);
    return hipGetLastError();
  }
  if (nblk > 0) {
    hipLaunchKernelGGL(expert_hist_kernel, dim3(nblk), dim3(PERM_BLOCK), lds, st, tok_off, ids, T, E,
                       block_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  int Q = 1;  // threads per expert in the scan: a power of two with Q * E <= 1024
  while (Q * 2 * E <= 1024) Q *= 2;
  // beyond 64 blocks per thread group the block sums move to one workgroup per expert
  const int presummed = nblk > 64 * Q ? 1 : 0;
  if (presummed) {
    hipLaunchKernelGGL(expert_block_scan_kernel, dim3(E), dim3(256), 0, st, block_counts, nblk, E, block_base, counts);
    hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
  }
  hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, st, block_counts, nblk, E, Q, block_base, counts,
                     expert_off, n_active, stats, RB, bound, blocks, presummed);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  hipLaunchKernelGGL(expert_scatter_kernel, dim3(nblk * SCATTER_SPLIT), dim3(PERM_BLOCK), 2 * lds, st, tok_off, ids,
                     T, E, k_max, block_base, expert_off, perm_tok, perm_src, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
