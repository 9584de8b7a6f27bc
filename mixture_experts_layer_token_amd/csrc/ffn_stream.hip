// Weight-streaming grouped SwiGLU FFN on MFMA (the memory-bound decode path).
//
// In decode the layer's time is the time to load the activated experts'
// weights from HBM (METRO reading notes, arXiv 2512.09277, Q1; ExFold summary,
// arXiv 2608.24938, MoE Inference: decode is batch-memory bound), so every
// weight byte is read exactly once, with 16-byte loads, by one wave, while the
// few rows routed to that expert ride along on the narrow side of a 16x16 MFMA.
//
// Work split.  The rows of each expert group are cut into blocks of up to
// 64 rows, listed in a row-block table built on the device (entries past the
// real count are sentinels), so the grid -- column tiles x table bound --
// depends only on the layer shape and carries no per-expert slack: a
// workgroup takes one (row block, column tile) pair.  A workgroup is WN x WK
// waves: WN waves along the output columns, WK waves along K.  A wave owns TPW
// 16-row weight tiles:
//   gate/up: TPW/2 tiles of W_gate rows and the same rows of W_up
//   down:    TPW tiles of W_down rows
// and for each K step loads, per lane, KC contiguous elements of one weight
// row per tile (lane l: row l%16, K offset (l/16)*KC).  The activation rows use
// the same K indices on the other MFMA side, so the instruction sums exactly
// the K values the lanes supplied (any consistent K order gives the dot
// product).  A block of at most 32 rows is one row group: the WK waves split
// K and add their partial sums through LDS in a fixed order (deterministic).
// A block of 33..64 rows (and, when K is short, every block) runs the
// shared-tile body below: its weight tile passes through LDS once for all 64
// rows.  This matters because the 16-row x 64-byte pattern of the direct
// loads moves L2-resident data into a CU at well under half the rate of
// whole-line loads, and heavily used experts are read from the L2 by many row
// blocks.  (Workgroups of two waves along K per row group stand in where the
// shared body does not apply.)
//
// Memory pipeline: the weights of step i+1 are requested before the MFMAs of
// step i, right after the activation rows of step i, so the in-order wait for
// the activations leaves the next weights in flight.
//
// The gate/up epilogue applies SwiGLU (MoE-Prism, arXiv 2510.19366, §III-B1,
// Eq. (1)): H = SiLU(g) * u, stored in the element type.
#include "common.h"
#include "launch.h"

namespace moe {

template <typename T, bool NT>
__device__ __forceinline__ uint4 ldw(const T* p) {
  if (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
__device__ __forceinline__ uint4 ld16(const T* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
__device__ __forceinline__ void mma_tile(f32x4_t& acc, const uint4& a, const uint4& b);

template <>
__device__ __forceinline__ void mma_tile<bf16_t>(f32x4_t& acc, const uint4& a, const uint4& b) {
  acc = Mfma<bf16_t>::step(a, b, acc);
}

template <>
__device__ __forceinline__ void mma_tile<float>(f32x4_t& acc, const uint4& a, const uint4& b) {
  acc = mfma_f32_4(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = mfma_f32_4(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = mfma_f32_4(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = mfma_f32_4(__uint_as_float(a.w), __uint_as_float(b.w), acc);
}

// Four consecutive outputs of a row.  Non-temporal stores: the next kernel
// reads H or Y once, and ordinary stores interleaved with the weight stream
// slowed it (see the grouped GEMM's epilogue).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  u32x2_t v;
  v.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  v.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4_t v;
  v.x = a;
  v.y = b;
  v.z = c;
  v.w = d;
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// MODE 0: gate/up + SwiGLU.  MODE 1: down projection.
// TPW: 16-row weight tiles per wave.  MODE 0: TPW/2 column tiles of W_gate and
// the same columns of W_up; MODE 1: TPW column tiles of W_down.  More tiles
// per wave put more weight bytes in flight per activation row loaded.
// IL: K layout of a lane's LPS 16-byte loads within a step.  IL = 0: load i of
// lane group g covers [g*KC + i*LE, +LE) (each lane reads KC contiguous
// elements); IL = 1: [i*4*LE + g*LE, +LE) (the four lane groups of one load
// read 64 contiguous bytes of the row).
// PD: software-pipeline depth.  The weights and activation rows of step s+PD
// are requested together before the MFMAs of step s, always with the same
// number of loads per step, so the in-order wait for step s leaves PD steps in
// flight.
// SM: 16-row activation tiles per pass (the block's rows; a block of at most
// 16 rows runs the SM = 1 body, which loads half the activation bytes).
// WKR: waves splitting K within this wave's row group; wk: this wave's index
// among them; slot0: the group's first LDS reduction slot; SLOT: f32x4 per slot.
template <typename T, int MODE, int KC, int WN, int WKR, int SM, int TPW, int PD, bool IL, int SLOT>
__device__ __forceinline__ void stream_block(const T* __restrict__ in, const int32_t* __restrict__ row_map,
                                             const T* wa, const T* wb, int K, int kbeg, int lofs, int nsteps,
                                             int mg, int rows, T* __restrict__ out, int N, int n0, f32x4_t* red,
                                             int wn, int wk, int slot0, int tstride, int kstr) {
  constexpr int LE = 16 / sizeof(T);                     // elements per 16-byte load
  constexpr int LPS = KC / LE;                           // loads per tile row per K step
  constexpr int STEP = 4 * KC;                           // K elements per wave step
  constexpr int NS = PD + 1;                             // register stages
  constexpr int LSTR = IL ? 4 * LE : LE;                 // distance between a lane's loads
  constexpr int HALF = TPW / 2;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // tile j's row pointer is wbase(j) + (j % half) * tstride (tstride: weight
  // elements between consecutive 16-row tiles; kstr: between consecutive
  // steps of K, both set by the weight layout)
  auto wrow = [&](int j) -> const T* {
    if (MODE == 0) return (j < HALF ? wa : wb) + (j % HALF) * tstride;
    return wa + j * tstride;
  };
  (void)wb;

  const int mts = (rows + 15) >> 4;  // live row tiles (wave-uniform)
  const T* xr[SM];
  bool valid[SM];
#pragma unroll
  for (int mt = 0; mt < SM; ++mt) {
    const int r = mt * 16 + lr;
    valid[mt] = r < rows;
    const int src = valid[mt] ? (row_map ? row_map[mg + r] : mg + r) : 0;
    xr[mt] = in + (size_t)src * K + kbeg + lofs;
  }
#pragma unroll
  for (int mt = 1; mt < SM; ++mt)
    if (mt >= mts) xr[mt] = xr[0];  // dead row tile: same loads as tile 0, result unused
  f32x4_t acc[SM][TPW];
#pragma unroll
  for (int mt = 0; mt < SM; ++mt)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[mt][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 Wr[NS][TPW][LPS];
  uint4 Xr[NS][SM][LPS];
  auto issue = [&](uint4 (&w)[TPW][LPS], uint4 (&x)[SM][LPS], int step) {
    const int ko = step * STEP, kw = step * kstr;
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int i = 0; i < LPS; ++i) w[j][i] = ldw<T, false>(wrow(j) + kw + i * LSTR);
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
#pragma unroll
      for (int i = 0; i < LPS; ++i) x[mt][i] = ld16(xr[mt] + ko + i * LSTR);
  };
#pragma unroll
  for (int p = 0; p < PD; ++p) issue(Wr[p], Xr[p], min(p, nsteps - 1));

  for (int s0 = 0; s0 < nsteps; s0 += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int s = s0 + st;
      if (s < nsteps) {
        // requests for step s + PD (the last step repeats: cached, in bounds)
        issue(Wr[(st + PD) % NS], Xr[(st + PD) % NS], min(s + PD, nsteps - 1));
#pragma unroll
        for (int mt = 0; mt < SM; ++mt)
          if (mt < mts) {
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
              const uint4 b = valid[mt] ? Xr[st][mt][i] : zero_u4();
#pragma unroll
              for (int j = 0; j < TPW; ++j) mma_tile<T>(acc[mt][j], Wr[st][j][i], b);
            }
          }
      }
    }
  }

  if (WKR > 1) {
    if (wk > 0) {
      f32x4_t* r = red + (size_t)((slot0 + wk - 1) * WN + wn) * SLOT;
#pragma unroll
      for (int mt = 0; mt < SM; ++mt)
#pragma unroll
        for (int j = 0; j < TPW; ++j) r[(mt * TPW + j) * 64 + lane] = acc[mt][j];
    }
    __syncthreads();
    if (wk == 0) {
      for (int q = 1; q < WKR; ++q) {
        const f32x4_t* r = red + (size_t)((slot0 + q - 1) * WN + wn) * SLOT;
#pragma unroll
        for (int mt = 0; mt < SM; ++mt)
#pragma unroll
          for (int j = 0; j < TPW; ++j) acc[mt][j] += r[(mt * TPW + j) * 64 + lane];
      }
    }
  }

  if (wk == 0) {
#pragma unroll
    for (int mt = 0; mt < SM; ++mt) {
      const int m = mt * 16 + lr;
      if (mt < mts && m < rows) {
        T* orow = out + (size_t)(mg + m) * N + n0 + 4 * lg;
        if (MODE == 0) {
#pragma unroll
          for (int j = 0; j < HALF; ++j) {
            const f32x4_t gt = acc[mt][j], up = acc[mt][j + HALF];
            store4<T>(orow + 16 * j, silu(gt[0]) * up[0], silu(gt[1]) * up[1], silu(gt[2]) * up[2],
                      silu(gt[3]) * up[3]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            const f32x4_t y = acc[mt][j];
            store4<T>(orow + 16 * j, y[0], y[1], y[2], y[3]);
          }
        }
      }
    }
  }
}

// Shared-tile body for a block of 33..64 rows in a workgroup of four waves
// along K (WN = 1).  Each K step of the workgroup -- the TPW = 4 weight tiles
// (16 rows x 128 bytes each) and the block's 64 activation rows (128 bytes
// each) -- is copied into LDS by global->LDS DMA loads of whole 128-byte
// lines (wave w fetches weight tile w and activation rows 16w..16w+15), two
// steps ahead in a ring of three stages (or more, VAR below).  Every wave then multiplies all four
// weight tiles with its own 16 activation rows and runs over the whole K, so
// there is no reduction.  The weights of such a block leave the L2 once, as
// full lines, instead of once per 32-row half as 64-byte half lines.  With no
// register loads in the loop, every wait is an explicit count.
// `ring` holds 3 stages of 16 KB: [weights 64 x 128 B][activations 64 x 128 B].
constexpr int SHARED_STAGE_BYTES = 2 * 64 * 128;
// VAR bits 2-3: extra ring stages (3 + n stages, n + 2 steps ahead).
// VAR bit 4: a two-stage ring instead (one step ahead; 32 KB of LDS).
template <int VAR> constexpr int shared_stages() { return (VAR & 16) ? 2 : 3 + ((VAR >> 2) & 3); }

// VAR bit 1: the weight DMA carries the non-temporal hint (the weights are
// read once per layer).
template <typename T, int MODE, int KC, int TPW, int VAR = 0>
__device__ __forceinline__ void stream_block_shared(const T* __restrict__ in, const int32_t* __restrict__ row_map,
                                                    const T* w0, const T* w1, int K, int mg, int rows,
                                                    T* __restrict__ out, int N, int n0, char* ring, int blocked) {
  constexpr int LE = 16 / sizeof(T);
  constexpr int LPS = KC / LE;
  constexpr int STEP = 4 * KC;
  constexpr int HALF = TPW / 2;
  constexpr int NST = shared_stages<VAR>(), AHEAD = NST - 1;
  constexpr int SB = SHARED_STAGE_BYTES, XOFS = SB / 2;
  static_assert(STEP * sizeof(T) == 128 && LPS == 2, "a step is one 128-byte line per row");
  static_assert(TPW == 4, "one weight tile and 16 activation rows per wave");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int nsteps = K / STEP;

  // DMA instruction q of wave w fills LDS rows 16w + 8q .. +7 of the weight
  // and the activation region (1 KB each); lane i writes chunk slot i % 8 of
  // row R = 16w + 8q + i / 8 and so fetches K chunk (i % 8) ^ swz(R).
  const T* tb = MODE == 0 ? (wave < HALF ? w0 : w1) : w0;
  const int trow = MODE == 0 ? n0 + 16 * (wave % HALF) : n0 + 16 * wave;  // first row of this wave's tile
  const int kstr = blocked ? w_kstep<T>(1) : STEP;                         // weight elements per step
  // Activation rows past the block's end: an instruction whose eight rows
  // are all missing is not issued (wave-uniform); within a partly filled one
  // a missing row repeats the block's first row (its outputs are not stored).
  const T* wsrc[2];
  const T* xsrc[2];
  bool xon[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * q + (lane >> 3), R = 16 * wave + r;
    const int c = (lane & 7) ^ lds_swz(R);
    wsrc[q] = tb + w_offset<T>(trow + r, c * LE, K, blocked);
    xon[q] = 16 * wave + 8 * q < rows;
    const int m = R < rows ? R : 0;
    const int src = row_map ? row_map[mg + m] : mg + m;
    xsrc[q] = in + (size_t)src * K + c * LE;
  }
  const int per_step = 2 + (xon[0] ? 1 : 0) + (xon[1] ? 1 : 0);  // loads this wave issues per step
  auto issue = [&](int s) {
    char* sb = ring + (s % NST) * SB + wave * 2048;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wsrc[q] + s * kstr), (lds_ptr_t)(sb + q * 1024), 16, 0,
                                       (VAR & 2) ? 2 : 0);
      if (xon[q])
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(xsrc[q] + s * STEP), (lds_ptr_t)(sb + XOFS + q * 1024), 16, 0,
                                         0);
    }
  };
  f32x4_t acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every step issues the same loads (past the end, the last step again: in
  // bounds, into a stage nobody reads any more), so the counts are constant.
#pragma unroll
  for (int p = 0; p < AHEAD; ++p) issue(min(p, nsteps - 1));
  for (int s = 0; s < nsteps; ++s) {
    // step s landed for this wave (steps s + 1 .. s + AHEAD - 1 may be in
    // flight); after the barrier every wave's part has landed and every wave
    // is done reading the stage that step s + AHEAD refills
    vm_wait_dyn<4 * (AHEAD - 1)>((AHEAD - 1) * per_step);
    lgkm_wait0();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    issue(min(s + AHEAD, nsteps - 1));
    const char* sb = ring + (s % NST) * SB;
    uint4 W[TPW][LPS], X[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      X[i] = *reinterpret_cast<const uint4*>(sb + XOFS + lds_off(16 * wave + lr, lg + 4 * i));
#pragma unroll
      for (int j = 0; j < TPW; ++j) W[j][i] = *reinterpret_cast<const uint4*>(sb + lds_off(16 * j + lr, lg + 4 * i));
    }
#pragma unroll
    for (int i = 0; i < LPS; ++i)
#pragma unroll
      for (int j = 0; j < TPW; ++j) mma_tile<T>(acc[j], W[j][i], X[i]);
  }
  vm_wait<0>();  // no DMA into LDS may outlive the workgroup

  const int m = 16 * wave + lr;
  if (m < rows) {
    T* orow = out + (size_t)(mg + m) * N + n0 + 4 * lg;
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const f32x4_t gt = acc[j], up = acc[j + HALF];
        store4<T>(orow + 16 * j, silu(gt[0]) * up[0], silu(gt[1]) * up[1], silu(gt[2]) * up[2],
                  silu(gt[3]) * up[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TPW; ++j) store4<T>(orow + 16 * j, acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
  }
}

// Linear workgroup id = block * tiles + tile.  Workgroups are dealt to the
// XCDs round-robin by linear id, so when the tile count is a multiple of 8 all
// row blocks of one column tile (an expert with many rows has several) run
// on the same XCD and share its L2 copy of the weight tile.  Blocks hold up to
// 32*SMT rows (two row groups of 16*SMT).  OCC: waves per SIMD the register
// allocation must allow (1: no constraint).
// VAR (shared-tile configurations only): bit 0 runs every block through the
// shared-tile body (the direct body is then not compiled in, which also frees
// its registers); bit 1 as in stream_block_shared.
// DENSE: one dense group of dense_rows rows (the always-on shared expert;
// blocks is then NULL); a separate instantiation, so that profiles list
// those launches apart from the routed ones.
// SEC: the launch also carries a second, dense problem of the same N and K
// (rows [0, rows_s) of in_s, no row map, weights w0s / w1s, into out_s: the
// always-on shared expert) as its first blocks, before the routed table's
// entries.  Its blocks hold 64 rows each, against a few rows in a routed
// block, so they are the launch's longest items and go out first: with them
// last, their items ran on after the routed stream had drained (128 tokens,
// 256 experts, d = 7168, a 2048-wide shared expert: 3.18 against 3.21 ms
// per layer, and 3.21 ms with the shared expert in launches of its own).
template <typename T, int MODE, int KC, int WN, int WK, int SMT, int TPW, int PD, bool IL, int OCC, int VAR = 0,
          bool DENSE = false, bool SEC = false>
__global__ __launch_bounds__(64 * WN * WK) __attribute__((amdgpu_waves_per_eu(OCC, 8))) void ffn_stream_kernel(
    const T* __restrict__ in, const int32_t* __restrict__ row_map, const T* __restrict__ w0,
    const T* __restrict__ w1, const int4* __restrict__ blocks, int dense_rows, T* __restrict__ out, int N, int K,
    int tiles, int blocked, const T* __restrict__ in_s, const T* __restrict__ w0s, const T* __restrict__ w1s,
    T* __restrict__ out_s, int rows_s) {
  if (DENSE) blocks = nullptr;
  static_assert(MODE == 1 || TPW % 2 == 0, "gate/up tiles come in pairs");
  static_assert(KC % (16 / sizeof(T)) == 0, "K step must be whole 16-byte loads");
  static_assert(WK % 2 == 0, "two row groups split the K waves in halves");
  constexpr int CPW = (MODE == 0) ? 8 * TPW : 16 * TPW;  // output columns per wave
  constexpr int NB = WN * CPW;                           // output columns per workgroup
  constexpr int LE = 16 / sizeof(T);
  constexpr int STEP = 4 * KC;                           // K elements per wave step
  constexpr int GR = 16 * SMT;                           // rows per row group
  constexpr int SLOT = SMT * TPW * 64;                   // f32x4 per reduction slot
  // shared-tile mode for 33..64-row blocks (see stream_block_shared)
  constexpr bool SHARED = WN == 1 && WK == 4 && TPW == 4 && IL && KC * sizeof(T) == 32;
  constexpr int RED_BYTES = (WK - 1) * WN * SLOT * (int)sizeof(f32x4_t);
  constexpr int RING_BYTES = shared_stages<VAR>() * SHARED_STAGE_BYTES;
  constexpr int LDS_BYTES = SHARED && RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  f32x4_t* const red = reinterpret_cast<f32x4_t*>(smem);

  int blk = blockIdx.x / tiles;
  const int tile = blockIdx.x - blk * tiles;
  const int nblk_s = SEC ? (rows_s + 2 * GR - 1) / (2 * GR) : 0;
  int g, mg, rows;  // group, first row of the block, rows in the block
  if (SEC && blk < nblk_s) {
    g = 0;
    mg = blk * 2 * GR;
    rows = min(2 * GR, rows_s - mg);
    in = in_s;
    row_map = nullptr;
    w0 = w0s;
    w1 = w1s;
    out = out_s;
  } else if (blocks) {
    if (SEC) blk -= nblk_s;
    const int4 b = blocks[blk];
    g = b.x;
    mg = b.y;
    rows = b.z;
    if (g < 0) return;
  } else {
    g = 0;
    mg = blk * 2 * GR;
    rows = min(2 * GR, dense_rows - mg);
    if (rows <= 0) return;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % WN, wk = wave / WN;
  const int lg = lane >> 4, lr = lane & 15;
  const int n0 = tile * NB + wn * CPW;
  const int lofs = IL ? lg * LE : lg * KC;   // lane's first element within a step
  const size_t gstride = (size_t)N * K;
  // A wave's rows n0 .. n0 + CPW - 1 lie in one 64-row block of the blocked
  // layout (n0 is a multiple of CPW), and each K step is one EB-wide column
  // of blocks (STEP = EB), so both layouts are plain pointer strides here.
  static_assert(STEP * sizeof(T) == 128 && 64 % CPW == 0, "layout strides");
  const size_t wofs = w_offset<T>(n0 + lr, lofs, K, blocked);
  const T* const wrow_a = w0 + g * gstride + wofs;
  const T* const wrow_b = (MODE == 0 ? w1 : w0) + g * gstride + wofs;
  const int tstride = (int)w_rowstep<T>(16, K, blocked), kstr = blocked ? w_kstep<T>(1) : STEP;
  // With a short K (under four steps per wave when split WK ways) every
  // block takes the shared-tile body, whose waves each run the whole K.
  const int light_max = !SHARED ? GR : ((VAR & 1) ? 0 : (K / WK / STEP >= 4 ? GR : 0));
  if (rows <= light_max) {
    // one row group; the WK waves split K
    const int Kw = K / WK, kbeg = wk * Kw, nsteps = Kw / STEP;
    const size_t kw0 = w_offset<T>(0, kbeg, K, blocked);
    if (SMT > 1 && rows <= 16)
      stream_block<T, MODE, KC, WN, WK, 1, TPW, PD, IL, SLOT>(in, row_map, wrow_a + kw0, wrow_b + kw0, K, kbeg, lofs,
                                                              nsteps, mg, rows, out, N, n0, red, wn, wk, 0, tstride, kstr);
    else
      stream_block<T, MODE, KC, WN, WK, SMT, TPW, PD, IL, SLOT>(in, row_map, wrow_a + kw0, wrow_b + kw0, K, kbeg,
                                                                lofs, nsteps, mg, rows, out, N, n0, red, wn, wk, 0, tstride, kstr);
  } else if constexpr (SHARED) {
    stream_block_shared<T, MODE, KC, TPW, VAR>(in, row_map, w0 + g * gstride, (MODE == 0 ? w1 : w0) + g * gstride, K, mg,
                                          rows, out, N, n0, smem, blocked);
  } else {
    // two row groups; WK/2 waves split K within each
    constexpr int WKR = WK / 2;
    const int grp = wk / WKR, wkr = wk - grp * WKR;
    const int Kw = K / WKR, kbeg = wkr * Kw, nsteps = Kw / STEP;
    const size_t kw0 = w_offset<T>(0, kbeg, K, blocked);
    const int mgg = mg + grp * GR, rg = min(GR, rows - grp * GR);
    if (SMT > 1 && rg <= 16)
      stream_block<T, MODE, KC, WN, WKR, 1, TPW, PD, IL, SLOT>(in, row_map, wrow_a + kw0, wrow_b + kw0, K, kbeg,
                                                               lofs, nsteps, mgg, rg, out, N, n0, red, wn, wkr,
                                                               grp * (WKR - 1), tstride, kstr);
    else
      stream_block<T, MODE, KC, WN, WKR, SMT, TPW, PD, IL, SLOT>(in, row_map, wrow_a + kw0, wrow_b + kw0, K, kbeg,
                                                                 lofs, nsteps, mgg, rg, out, N, n0, red, wn, wkr,
                                                                 grp * (WKR - 1), tstride, kstr);
  }
}

// Shape rules a launch must satisfy (checked by the callers): N % NB == 0,
// K % WK == 0, (K / WK) % (4 * KC) == 0.
template <typename T, int MODE, int KC, int WN, int WK, int SMT, int TPW, int PD, bool IL = true, int OCC = 1>
constexpr int stream_nb() { return WN * ((MODE == 0) ? 8 * TPW : 16 * TPW); }

template <typename T, int MODE, int KC, int WN, int WK, int SMT, int TPW, int PD, bool IL = true, int OCC = 1,
          int VAR = 0>
hipError_t launch_stream_variant(const T* in, const int32_t* row_map, const T* w0, const T* w1, const int4* blocks,
                                 int nblk, int dense_rows, T* out, int N, int K, int blocked, hipStream_t st,
                                 const GemmSecond& sec) {
  constexpr int NB = stream_nb<T, MODE, KC, WN, WK, SMT, TPW, PD, IL, OCC>();
  const int tiles = N / NB;
  const int nblk_s = (blocks && sec.rows > 0) ? (sec.rows + 32 * SMT - 1) / (32 * SMT) : 0;  // 2 x 16 SMT rows per block
  const long long total = (long long)tiles * (nblk + nblk_s);
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL / (64 * WN * WK)) return hipErrorInvalidValue;
  if (nblk_s > 0)
    hipLaunchKernelGGL((ffn_stream_kernel<T, MODE, KC, WN, WK, SMT, TPW, PD, IL, OCC, VAR, false, true>),
                       dim3((unsigned)total), dim3(64 * WN * WK), 0, st, in, row_map, w0, w1, blocks, dense_rows, out,
                       N, K, tiles, blocked, (const T*)sec.in, (const T*)sec.w0, (const T*)sec.w1, (T*)sec.out,
                       sec.rows);
  else if (blocks)
    hipLaunchKernelGGL((ffn_stream_kernel<T, MODE, KC, WN, WK, SMT, TPW, PD, IL, OCC, VAR, false>), dim3((unsigned)total),
                       dim3(64 * WN * WK), 0, st, in, row_map, w0, w1, blocks, dense_rows, out, N, K, tiles, blocked,
                       nullptr, nullptr, nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((ffn_stream_kernel<T, MODE, KC, WN, WK, SMT, TPW, PD, IL, OCC, VAR, true>), dim3((unsigned)total),
                       dim3(64 * WN * WK), 0, st, in, row_map, w0, w1, blocks, dense_rows, out, N, K, tiles, blocked,
                       nullptr, nullptr, nullptr, nullptr, 0);
  return hipGetLastError();
}

// Production shape of the streaming kernels (chosen by sweeps over tile
// shapes on the decode workloads): 16-element K chunks per lane (a 64-element
// step per wave), four 16-row weight tiles per wave, 64 rows per block, and
// the four waves of a workgroup splitting K.  When K/4 is not a whole number
// of steps the workgroup is 2 x 2 waves.  Pipeline depth: one step ahead; two
// in bf16 when every wave runs at least 16 steps (long K, e.g. the down
// projection of a 14336-wide expert), where the deeper queue outweighs the
// lower occupancy its registers cost (3 -> 2 waves per SIMD); with short K
// the prologue dominates and the deeper pipeline loses.
constexpr int S_SMT = 2, S_TPW = 4;
constexpr int S_ROWS = 32 * S_SMT;   // rows per block (two row groups)
constexpr int S_DEEP_STEPS = 16;     // steps per wave from which bf16 runs two steps ahead

int stream_row_block() { return S_ROWS; }

// Body and cache hint of the bf16 1 x 4-wave kernel (VAR above), from
// interleaved timings on the decode shapes: the shared-tile body with
// non-temporal weight DMA streams the gate/up pair faster unless the expert
// is very wide (N >= 8192: Mixtral-shaped, 332 vs 343 us) -- DSV3-shaped
// 2272 -> 2014 us, Qwen3-shaped 83 -> 75 us -- and the down projection of a
// long K (>= 8192: 165 -> 139 us); a short-K down projection (K <= 1024)
// gains from the shared body alone (37 -> 32 us); others keep the mix.
// With blocked weights every tile step is one contiguous 2 KB run, and the
// shared body with the hint wins everywhere (Mixtral-shaped gate/up 331 ->
// 295 us, DSV3-shaped down 1116 -> 1029 us, Qwen3-shaped gate/up 76 -> 73
// us).  Timed with a 1 GiB cache-evicting write before every launch (as in a
// model, where the other layers' weights pass through the 256 MB last-level
// cache between two calls of one layer), the short-K down projection keeps
// the hint too: Qwen3-shaped, K = 768, 79 us without it, 47 us with it (warm,
// without the write, its weights stay in that cache and the plain loads win:
// 36 vs 43 us).  A down projection of mid-size K (DSV3-shaped, K = 2048)
// gains from a ring one stage deeper (1049 -> 1031 us), which the others do
// not (Mixtral-shaped down 152 vs 154 us, Qwen3-shaped down 47 vs 49 us,
// gate/up 305 vs 333 us: two workgroups per CU instead of three).  The other
// way, a two-stage ring (32 KB: five workgroups per CU instead of three) wins
// for a gate/up pair where both N and K are at most 2048, i.e. many short
// items: Qwen3-shaped gate/up 76 -> 71 us, layer 0.1605 -> 0.1578 ms, and
// 0.1547 ms with its down projection (K = 768) left on three stages; it
// loses on the long streams (Mixtral-shaped layer +10 %, DSV3-shaped decode
// +1 %).
static int stream_var(int MODE, int N, int K, int blocked) {
  if (blocked && MODE == 0 && N <= 2048 && K <= 2048) return 19;
  if (blocked) return MODE == 0 ? 3 : ((K > 1024 && K < 8192) ? 7 : 3);
  if (MODE == 0) return N >= 8192 ? 0 : 3;
  if (K >= 8192) return 3;
  return K <= 1024 ? 1 : 0;
}

template <typename T, int MODE, int WN, int WK, int PD>
static hipError_t stream_pd(const T* x, const int32_t* row_map, const T* w0, const T* w1, const int4* blocks,
                            int nblk, int dense_rows, T* out, int N, int K, int blocked, hipStream_t st,
                            const GemmSecond& sec) {
  constexpr int KC = (sizeof(T) == 2) ? 16 : 8;
  if constexpr (sizeof(T) == 2 && WN == 1 && WK == 4) {
    switch (stream_var(MODE, N, K, blocked)) {
      case 3:
        return launch_stream_variant<T, MODE, KC, WN, WK, S_SMT, S_TPW, PD, true, 1, 3>(x, row_map, w0, w1, blocks,
                                                                                     nblk, dense_rows, out, N, K, blocked, st, sec);
      case 19:
        return launch_stream_variant<T, MODE, KC, WN, WK, S_SMT, S_TPW, PD, true, 1, 19>(x, row_map, w0, w1, blocks,
                                                                                      nblk, dense_rows, out, N, K, blocked, st, sec);
      case 7:
        return launch_stream_variant<T, MODE, KC, WN, WK, S_SMT, S_TPW, PD, true, 1, 7>(x, row_map, w0, w1, blocks,
                                                                                     nblk, dense_rows, out, N, K, blocked, st, sec);
      case 1:
        return launch_stream_variant<T, MODE, KC, WN, WK, S_SMT, S_TPW, PD, true, 1, 1>(x, row_map, w0, w1, blocks,
                                                                                     nblk, dense_rows, out, N, K, blocked, st, sec);
      default:
        break;
    }
  }
  return launch_stream_variant<T, MODE, KC, WN, WK, S_SMT, S_TPW, PD>(x, row_map, w0, w1, blocks, nblk, dense_rows,
                                                                      out, N, K, blocked, st, sec);
}

template <typename T, int MODE, int WN, int WK>
static hipError_t stream_wk(const T* x, const int32_t* row_map, const T* w0, const T* w1, const int4* blocks,
                            int nblk, int dense_rows, T* out, int N, int K, int blocked, hipStream_t st,
                            const GemmSecond& sec) {
  constexpr int KC = (sizeof(T) == 2) ? 16 : 8;
  constexpr int STEP = 4 * KC;
  if constexpr (sizeof(T) == 2) {
    if (K / WK / STEP >= S_DEEP_STEPS)
      return stream_pd<T, MODE, WN, WK, 2>(x, row_map, w0, w1, blocks, nblk, dense_rows, out, N, K, blocked, st, sec);
  }
  return stream_pd<T, MODE, WN, WK, 1>(x, row_map, w0, w1, blocks, nblk, dense_rows, out, N, K, blocked, st, sec);
}

template <typename T, int MODE>
static hipError_t stream_t(const void* in, const int32_t* row_map, const void* w0, const void* w1, const int4* blocks,
                           int bound, int dense_rows, void* out, int N, int K, int blocked, hipStream_t st,
                           const GemmSecond& sec) {
  constexpr int KC = (sizeof(T) == 2) ? 16 : 8;
  constexpr int STEP = 4 * KC;
  const int nblk = blocks ? bound : (dense_rows + S_ROWS - 1) / S_ROWS;
  const T* x = (const T*)in;
  if (K % (4 * STEP) == 0)
    return stream_wk<T, MODE, 1, 4>(x, row_map, (const T*)w0, (const T*)w1, blocks, nblk, dense_rows, (T*)out, N, K, blocked, st, sec);
  return stream_wk<T, MODE, 2, 2>(x, row_map, (const T*)w0, (const T*)w1, blocks, nblk, dense_rows, (T*)out, N, K, blocked, st, sec);
}

hipError_t launch_ffn_gateup_stream(int dtype, const void* in, const int32_t* row_map, const void* wg,
                                    const void* wu, const int4* blocks, int bound, int dense_rows, void* h, int N,
                                    int K, int blocked, hipStream_t st, const GemmSecond& sec) {
  if (dtype == DT_BF16)
    return stream_t<bf16_t, 0>(in, row_map, wg, wu, blocks, bound, dense_rows, h, N, K, blocked, st, sec);
  return stream_t<float, 0>(in, row_map, wg, wu, blocks, bound, dense_rows, h, N, K, blocked, st, sec);
}

hipError_t launch_ffn_down_stream(int dtype, const void* h, const int32_t* row_map, const void* wd,
                                  const int4* blocks, int bound, int dense_rows, void* y, int N, int K, int blocked,
                                  hipStream_t st, const GemmSecond& sec) {
  if (dtype == DT_BF16)
    return stream_t<bf16_t, 1>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K, blocked, st, sec);
  return stream_t<float, 1>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K, blocked, st, sec);
}

}  // namespace moe
