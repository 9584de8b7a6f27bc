// Grouped SwiGLU FFN as an LDS-tiled GEMM on bf16 MFMA (the compute-bound
// prefill path).
//
// With hundreds of rows per expert the expert FFN is a dense contraction
// (MoE-Prism, arXiv 2510.19366, §II-A: the k assignments per token scale the
// routed-expert GEMM volume; ExFold summary, arXiv 2608.24938: prefill is
// token-compute bound).  Each expert's rows are contiguous in the permuted
// order, so the layer is a grouped GEMM over experts:
//   gate/up: [rows_e, d] x [W_gate[e]; W_up[e]]^T, epilogue H = SiLU(g) * u
//            (MoE-Prism §III-B1, Eq. (1)), input rows gathered through perm_tok;
//   down:    [rows_e, I] x W_down[e]^T.
//
// Tiling: a workgroup (4 waves, 2 x 2) owns BM rows x BN columns of each of
// NMAT weight matrices (NMAT = 2 for the gate/up pair, 1 for down).  K advances
// BK = 64 at a time through double-buffered LDS (one barrier per step; the next
// step's global loads are in flight during the MFMAs).  A wave holds
// (BM/2) x (BN/2) outputs per matrix as 16x16 tiles of v_mfma_f32_16x16x32_bf16
// with the weights as the A operand, so a lane ends with 4 consecutive output
// columns of one row (8-byte stores).  LDS rows are padded by 16 bytes so the
// 16 rows a fragment read touches fall in distinct banks.
//
// Scheduling: the tiles of expert e are the row blocks [tile_off[e],
// tile_off[e+1]) (tile_off is built on the device from the per-expert counts),
// times the N tiles.  The grid is sized by an upper bound that depends only on
// the layer shape; each workgroup reads the real tile count and maps its id so
// that XCD x (ids x, x+8, ...) takes one contiguous range of (row block, N tile)
// pairs: the N tiles of a row block, then the next row block of the same
// expert, which keeps an expert's weights in that XCD's L2.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int GBM = 256;  // rows per row block of the tile table (a multiple of every BM used)
constexpr int GPAD = 8;   // LDS row padding (elements)

__device__ __forceinline__ void st_lds16(bf16_t* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ u32x4_t ld_lds16(const bf16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld_g16(const bf16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// MODE 0: gate/up pair + SwiGLU epilogue.  MODE 1: down projection.
// BM x BN (per weight matrix) output tile, BK K-elements per LDS stage,
// WGM x WGN waves.  BM must divide GBM (row blocks of the tile table).
template <int MODE, int BM, int BN, int BK, int WGM, int WGN, int PD>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_gemm_kernel(
    const bf16_t* __restrict__ in, const int32_t* __restrict__ row_map, const bf16_t* __restrict__ w0,
    const bf16_t* __restrict__ w1, const int32_t* __restrict__ grp_off, const int32_t* __restrict__ tile_off, int G,
    int dense_rows, bf16_t* __restrict__ out, int N, int K) {
  constexpr int NT = 64 * WGM * WGN;       // threads
  constexpr int NMAT = (MODE == 0) ? 2 : 1;
  constexpr int BROWS = NMAT * BN;         // weight rows staged per stage
  constexpr int LD = BK + GPAD;            // LDS row pitch (elements)
  constexpr int TM = BM / WGM / 16;        // 16-row tiles per wave
  constexpr int TN = BN / WGN / 16;        // 16-column tiles per wave per matrix
  constexpr int ACH = BM * BK / 8 / NT;    // 16-byte chunks of the row tile per thread
  constexpr int BCH = BROWS * BK / 8 / NT; // ... of the weight tile
  constexpr int SUB = GBM / BM;            // tiles per table row block
  static_assert(ACH >= 1 && BCH >= 1 && ACH * NT * 8 == BM * BK && BCH * NT * 8 == BROWS * BK, "chunking");
  static_assert(TM >= 1 && TN >= 1 && GBM % BM == 0, "tiling");
  __shared__ bf16_t As[2][BM * LD];
  __shared__ bf16_t Bs[2][BROWS * LD];

  // ---- which (group, row tile, N tile) this workgroup owns ----
  const int nN = N / BN;
  const int total_rb = grp_off ? tile_off[G] : (dense_rows + GBM - 1) / GBM;
  const int total = total_rb * SUB * nN;
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  if (slot >= per) return;
  const int logical = xcd * per + slot;
  if (logical >= total) return;
  const int mtile = logical / nN, nt = logical - mtile * nN;
  const int rb = mtile / SUB;
  int g = 0, row0 = 0, rows = dense_rows, mb = rb;
  if (grp_off) {
    int lo = 0, hi = G - 1;  // last g with tile_off[g] <= rb
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_off[mid] <= rb) lo = mid; else hi = mid - 1;
    }
    g = lo;
    row0 = grp_off[g];
    rows = grp_off[g + 1] - row0;
    mb = rb - tile_off[g];
  }
  const int m0 = mb * GBM + (mtile % SUB) * BM;  // first row of the tile within the group
  if (m0 >= rows) return;                        // the row block's rows end in an earlier sub-tile
  const int n0 = nt * BN;                        // first output column

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 15, lg = lane >> 4;

  // ---- global source pointers of this thread's 16-byte chunks ----
  const bf16_t* asrc[ACH];
  int adst[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + NT * i;
    const int r = c / (BK / 8), kc = c % (BK / 8);
    int m = m0 + r;
    if (m >= rows) m = rows - 1;                       // tail rows: any valid row, results unused
    const int src = row_map ? row_map[row0 + m] : row0 + m;
    asrc[i] = in + (size_t)src * K + kc * 8;
    adst[i] = r * LD + kc * 8;
  }
  const size_t gstride = (size_t)N * K;
  const bf16_t* bsrc[BCH];
  int bdst[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + NT * i;
    const int r = c / (BK / 8), kc = c % (BK / 8);
    const bf16_t* wbase = (MODE == 0 && r >= BN) ? w1 : w0;
    const int wr = (MODE == 0 && r >= BN) ? r - BN : r;
    bsrc[i] = wbase + g * gstride + (size_t)(n0 + wr) * K + kc * 8;
    bdst[i] = r * LD + kc * 8;
  }

  f32x4_t acc[TM][NMAT * TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < NMAT * TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Stage pipeline: LDS is double-buffered; the global loads of stage s + 1
  // are issued one stage ahead into one of two register sets used in turn
  // (the K loop is unrolled by two, so no set is ever copied).  K / BK is
  // even (K is a multiple of 128), and every iteration is the same
  // straight-line code -- a branch around the loads made the compiler keep the
  // registers in scratch: steps past the end re-read the last stage (cached)
  // and the final store goes to the idle buffer, which nobody reads.
  static_assert(PD == 1, "one stage of register prefetch");
  u32x4_t ra0[ACH], rb0[BCH], ra1[ACH], rb1[BCH];
  const int nk = K / BK;
#pragma unroll
  for (int i = 0; i < ACH; ++i) st_lds16(&As[0][adst[i]], ld_g16(asrc[i]));
#pragma unroll
  for (int i = 0; i < BCH; ++i) st_lds16(&Bs[0][bdst[i]], ld_g16(bsrc[i]));
  {
    const int k1 = min(1, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra0[i] = ld_g16(asrc[i] + k1);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb0[i] = ld_g16(bsrc[i] + k1);
  }
  __syncthreads();

  auto mma_stage = [&](const bf16_t* as, const bf16_t* bs) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t bfr[TM];   // activation rows: B operand
#pragma unroll
      for (int i = 0; i < TM; ++i) bfr[i] = ld_lds16(&as[(wm * (BM / WGM) + i * 16 + lr) * LD + kk + lg * 8]);
#pragma unroll
      for (int q = 0; q < NMAT * TN; ++q) {
        const int mat = q / TN, tj = q % TN;
        const u32x4_t afr = ld_lds16(&bs[(mat * BN + wn * (BN / WGN) + tj * 16 + lr) * LD + kk + lg * 8]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][q] = Mfma<bf16_t>::step(afr, bfr[i], acc[i][q]);
      }
    }
  };

  for (int kt = 0; kt < nk; kt += 2) {
    // even stage kt: LDS buffer 0; set 0 holds stage kt+1, set 1 receives kt+2
    {
      const int kn = min(kt + 2, nk - 1) * BK;
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra1[i] = ld_g16(asrc[i] + kn);
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb1[i] = ld_g16(bsrc[i] + kn);
    }
    mma_stage(As[0], Bs[0]);
#pragma unroll
    for (int i = 0; i < ACH; ++i) st_lds16(&As[1][adst[i]], ra0[i]);
#pragma unroll
    for (int i = 0; i < BCH; ++i) st_lds16(&Bs[1][bdst[i]], rb0[i]);
    __syncthreads();
    // odd stage kt+1: LDS buffer 1; set 1 holds kt+2, set 0 receives kt+3
    {
      const int kn = min(kt + 3, nk - 1) * BK;
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra0[i] = ld_g16(asrc[i] + kn);
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb0[i] = ld_g16(bsrc[i] + kn);
    }
    mma_stage(As[1], Bs[1]);
#pragma unroll
    for (int i = 0; i < ACH; ++i) st_lds16(&As[0][adst[i]], ra1[i]);
#pragma unroll
    for (int i = 0; i < BCH; ++i) st_lds16(&Bs[0][bdst[i]], rb1[i]);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[n = 4*lg + r][m = lr] of each 16x16 tile ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * (BM / WGM) + i * 16 + lr;
    if (m >= rows) continue;
    bf16_t* orow = out + (size_t)(row0 + m) * N + n0 + wn * (BN / WGN) + 4 * lg;
#pragma unroll
    for (int tj = 0; tj < TN; ++tj) {
      uint32_t o0, o1;
      if (MODE == 0) {
        const f32x4_t gt = acc[i][tj], up = acc[i][TN + tj];
        o0 = (uint32_t)f32_to_bf16(silu(gt[0]) * up[0]) | ((uint32_t)f32_to_bf16(silu(gt[1]) * up[1]) << 16);
        o1 = (uint32_t)f32_to_bf16(silu(gt[2]) * up[2]) | ((uint32_t)f32_to_bf16(silu(gt[3]) * up[3]) << 16);
      } else {
        const f32x4_t y = acc[i][tj];
        o0 = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
        o1 = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
      }
      *reinterpret_cast<uint2*>(orow + tj * 16) = make_uint2(o0, o1);
    }
  }
}

// tile_off[g] = sum over g' < g of ceil(rows_g' / GBM); one workgroup.
__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t* __restrict__ grp_off, int G,
                                                          int32_t* __restrict__ tile_off) {
  __shared__ int32_t sc[1024];
  const int g = threadIdx.x;
  int v = 0;
  if (g < G) v = (grp_off[g + 1] - grp_off[g] + GBM - 1) / GBM;
  sc[g] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = g >= off ? sc[g - off] : 0;
    __syncthreads();
    sc[g] += u;
    __syncthreads();
  }
  if (g < G) tile_off[g] = sc[g] - v;
  if (g == 1023) tile_off[G] = sc[1023];
}

int gemm_tile_bound(int A_cap, int G) { return (A_cap + GBM - 1) / GBM + G; }

template <int MODE, int BM, int BN, int BK, int WGM, int WGN, int PD>
hipError_t launch_gemm_variant(const void* in, const int32_t* row_map, const void* w0, const void* w1,
                               const int32_t* grp_off, const int32_t* tile_off, int G, int dense_rows, int rb_bound,
                               void* out, int N, int K, hipStream_t st) {
  const long long total = (long long)rb_bound * (GBM / BM) * (N / BN);
  if (total == 0) return hipSuccess;
  const long long blocks = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((ffn_gemm_kernel<MODE, BM, BN, BK, WGM, WGN, PD>), dim3((unsigned)blocks), dim3(64 * WGM * WGN), 0,
                     st, (const bf16_t*)in, row_map, (const bf16_t*)w0, (const bf16_t*)w1, grp_off, tile_off, G,
                     dense_rows, (bf16_t*)out, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm_tiles(const int32_t* grp_off, int G, int32_t* tile_off, hipStream_t st) {
  hipLaunchKernelGGL(gemm_tiles_kernel, dim3(1), dim3(1024), 0, st, grp_off, G, tile_off);
  return hipGetLastError();
}

hipError_t launch_ffn_gateup_gemm(const void* in, const int32_t* row_map, const void* wg, const void* wu,
                                  const int32_t* grp_off, const int32_t* tile_off, int G, int dense_rows,
                                  int rb_bound, void* h, int N, int K, hipStream_t st) {
  return launch_gemm_variant<0, 128, 64, 64, 2, 2, 1>(in, row_map, wg, wu, grp_off, tile_off, G, dense_rows, rb_bound,
                                                   h, N, K, st);
}

hipError_t launch_ffn_down_gemm(const void* h, const void* wd, const int32_t* grp_off, const int32_t* tile_off,
                                int G, int dense_rows, int rb_bound, void* y, int N, int K, hipStream_t st) {
  return launch_gemm_variant<1, 128, 128, 64, 2, 2, 1>(h, nullptr, wd, wd, grp_off, tile_off, G, dense_rows, rb_bound,
                                                    y, N, K, st);
}

}  // namespace moe
