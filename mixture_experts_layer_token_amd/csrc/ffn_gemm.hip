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
// Tiling.  A workgroup of WM x WN waves owns BM rows x BNW columns of each of
// NMAT weight matrices (NMAT = 2 for the gate/up pair, 1 for down).  K advances
// 64 at a time through a ring of STAGES LDS buffers filled by global->LDS DMA
// loads (global_load_lds_dwordx4): no VGPR staging, so the registers hold only
// accumulators and fragments, and the loads of the next stages are in flight
// while the current one is multiplied.  A wave holds (BM/WM) x (BNW/WN)
// outputs per matrix as 32x32 tiles of v_mfma_f32_32x32x16_bf16 with the
// weights as the A operand (a lane ends with 4 consecutive output columns of a
// row; the epilogue gathers the tile in LDS and stores whole lines).
//
// Weights are read row-major or in the blocked order (64-row x 128-byte
// blocks, w_offset in common.h): a lane's DMA source is set once, and a stage
// advances it by one row of 64 elements or by one whole 8 KB block.
//
// LDS layout.  A stage holds each tile row as 128 bytes (64 bf16 of K) with no
// padding; the eight 16-byte chunks of row r are XOR-permuted by (r >> 1) & 7.
// A DMA instruction writes 1 KB (64 lanes x 16 bytes) to consecutive LDS
// addresses, so the permutation is applied by choosing which global chunk each
// lane fetches.  With it, the fragment reads of the 32x32x16 MFMA (32 rows x
// two adjacent chunks per instruction) are free of bank conflicts on gfx950.
//
// Schedule.  Within a stage, the fragment reads of k16 step s+1 alternate with
// the MFMAs of step s (sched_group_barrier), so both fragment sets are live.
// The barrier that hands over stage kt+1 sits before the last k16 step of stage
// kt; after it the buffer of stage kt is refilled (stage kt+STAGES) and the
// first fragments of stage kt+1 are read during the last MFMAs of stage kt.
// One barrier per stage; the DMA waits are explicit vmcnt counts.
//
// Ring depth per operand.  The activation and weight parts of a stage live
// in rings of their own, XS and WS buffers deep.  The barrier of stage kt
// (after the wait for stage kt+1) frees buffer kt of both rings and issues
// x(kt+XS), then w(kt+WS); the prologue runs the same schedule for the
// virtual barriers -max(XS, WS) .. -1.  So the weights run WS-1 stages ahead
// and the gathered rows XS-1, and the wait for a stage counts exactly the
// DMA instructions issued after its later operand.  The 256-row tiles take
// XS = 2, WS = 3 (the 32 KB of LDS a two-stage ring leaves free holds a third
// weight buffer): sub-expert-shaped layer, bit-identical outputs, down 400 ->
// 377 us, gate/up 475 -> 462 us (rows deeper instead, XS = 3, WS = 2: 385 /
// 501).  NTW = 1 puts the non-temporal hint on the grouped problem's weight
// DMA (each routed expert's weights are read by one or two row tiles); the
// second problem's weights (re-read by all its row tiles) keep ordinary
// loads.
//
// Scheduling of tiles.  The rows of each expert are cut into row blocks of BM
// rows (the tile height) listed in a row-block table built on the device from
// the per-expert counts; a row block is one row tile, times the N tiles.  The
// grid is sized by the table's bound, which depends only on the layer shape;
// each workgroup reads the real block count and maps its id so that XCD x
// (ids x, x+8, ...) takes one contiguous range of (row tile, N tile) pairs:
// the N tiles of a row tile, then the next row tile of the same expert, which
// keeps an expert's weights and gathered rows in that XCD's L2.  (A persistent
// variant, one workgroup per CU running its tiles on one continuous DMA
// schedule with the epilogue overlapping the next tile's first stages, was
// bit-identical but slower: gate/up 2545 against 2500 us, 256 experts x 96
// rows, d = 7168, I = 2048; idle CUs between tiles do not cost bandwidth
// while the others stream.)
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int BK = 64;    // K elements per stage: one 128-byte LDS row per tile row

typedef float f32x16_t __attribute__((ext_vector_type(16)));
}  // namespace

// MODE 0: gate/up pair + SwiGLU epilogue.  MODE 1: down projection.
// XS, WS: ring depths of the activation and weight tiles.  NTW: non-temporal
// hint on the routed weights.  EPI: how the output tile is stored (0: from the
// fragments, gate/up only; 1: staged in LDS; 2: staged, non-temporal).  SEC:
// the launch carries the second, dense
// problem (rows_s > 0); a separate instantiation, so that profiles list the
// launches with the always-on expert's tiles apart from the routed-only ones.
template <int MODE, int BM, int BNW, int WM, int WN, int XS, int WS, int NTW = 0, int EPI = 1, bool SEC = false>
__global__ __launch_bounds__(64 * WM * WN) void ffn_gemm_kernel(
    const bf16_t* __restrict__ in, const int32_t* __restrict__ row_map, const bf16_t* __restrict__ w0,
    const bf16_t* __restrict__ w1, const int4* __restrict__ blocks, int bound, int dense_rows,
    bf16_t* __restrict__ out, int N, int K, const bf16_t* __restrict__ in_s, const bf16_t* __restrict__ w0s,
    const bf16_t* __restrict__ w1s, bf16_t* __restrict__ out_s, int rows_s, int blocked) {
  constexpr int NW = WM * WN;
  constexpr int NMAT = (MODE == 0) ? 2 : 1;
  constexpr int WROWS = NMAT * BNW;                          // weight rows per stage
  constexpr int XBYTES = BM * 128;
  constexpr int XI = BM / 8 / NW, WI = WROWS / 8 / NW;        // DMA instructions per wave per stage
  constexpr int TMW = BM / WM / 32, TNW = BNW / WN / 32;      // 32x32 tiles per wave
  constexpr int KS = BK / 16;                                 // k16 steps per stage
  static_assert(XI * 8 * NW == BM && WI * 8 * NW == WROWS, "DMA split");
  static_assert(TMW >= 1 && TNW >= 1, "tiling");
  static_assert(XS >= 2 && WS >= 2 && XS <= 4 && WS <= 4, "ring depths");
  constexpr int MAXS = XS > WS ? XS : WS, MINS = XS < WS ? XS : WS;
  // The epilogue stages the output tile here as well (rows of EPITCH bytes:
  // 16 bytes of padding keep the rows 16-byte aligned and spread the staging
  // writes over the banks).
  constexpr int EPITCH = BNW * 2 + 16;
  constexpr int WBYTES = WROWS * 128, RING = XS * XBYTES + WS * WBYTES;
  static_assert(RING <= 160 * 1024, "LDS");
  constexpr int LDS_BYTES = (EPI > 0 && BM * EPITCH > RING) ? BM * EPITCH : RING;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  // ---- which (row block, row tile, N tile) this workgroup owns.  In every
  // XCD's range the tiles of the second, dense problem (rows_s > 0: an
  // always-on expert over rows [0, rows_s) with weights w0s/w1s) come after
  // the grouped problem's in the gate/up launch, so these compute-bound tiles
  // (K = d) take the CUs that the end of the weight stream leaves idle (256
  // experts x 96 rows, d = 7168, a 4,096-row shared expert: 4.46 ms per layer
  // against 4.50-4.54 ms with the dense tiles spread evenly through the
  // grouped ones), and before them in the down launch, whose dense tiles are
  // short (K = I): 4.350 against 4.418 ms (three interleaved pairs). ----
  const int nN = N / BNW;
  const int r_mt = blocks ? blocks[bound].x : (dense_rows + BM - 1) / BM;
  const int s_mt = SEC ? (rows_s + BM - 1) / BM : 0;
  // XCD x (ids x, x + 8, ...) takes tiles [x * Rp, (x + 1) * Rp) of the
  // grouped problem, then tiles [x * Sp, (x + 1) * Sp) of the second one
  const int R = r_mt * nN, S2 = s_mt * nN, Rp = (R + 7) >> 3, Sp = (S2 + 7) >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  if (slot >= Rp + Sp) return;
  constexpr bool SFIRST = SEC && MODE == 1;  // the down projection's dense tiles lead its ranges
  const bool second = SEC && (SFIRST ? slot < Sp : slot >= Rp);
  const int li = second ? xcd * Sp + (SFIRST ? slot : slot - Rp) : xcd * Rp + (SFIRST ? slot - Sp : slot);
  if (li >= (second ? S2 : R)) return;
  const int mk = li / nN, nt = li - mk * nN;  // row tile within its problem, N tile
  const int rb = mk;
  int g, row0, rows;  // group, first row and rows of the row block
  if (second) {
    g = 0;
    row0 = rb * BM;
    rows = min(BM, rows_s - row0);
    in = in_s;
    row_map = nullptr;
    w0 = w0s;
    w1 = w1s;
    out = out_s;
  } else if (blocks) {
    const int4 b = blocks[rb];
    g = b.x;
    row0 = b.y;
    rows = b.z;
  } else {
    g = 0;
    row0 = rb * BM;
    rows = min(BM, dense_rows - row0);
  }
  const int n0 = nt * BNW;         // first output column

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- DMA sources.  Instruction j of this wave fills tile rows 8q .. 8q+7
  // (q = j*NW + wave); lane i covers row 8q + i/8, LDS chunk i%8, which holds
  // K chunk (i%8) ^ swz(row).  Rows past the group's end are not fetched
  // (their columns are never stored); the decision is made per instruction and
  // wave, so a wave issues the same count of DMA loads in every stage. ----
  const bf16_t* xsrc[XI];
  bool xon[XI], xany[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int r = 8 * (j * NW + wave) + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz(r);
    int m = r;
    xon[j] = m < rows;
    xany[j] = __builtin_amdgcn_ballot_w64(xon[j]) != 0;
    if (m >= rows) m = rows - 1;
    const int src = row_map ? row_map[row0 + m] : row0 + m;
    xsrc[j] = in + (size_t)src * K + c * 8;
  }
  const size_t gstride = (size_t)N * K;
  const bf16_t* wsrc[WI];
#pragma unroll
  for (int j = 0; j < WI; ++j) {
    const int r = 8 * (j * NW + wave) + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz(r);
    const bf16_t* wb = (MODE == 0 && r >= BNW) ? w1 : w0;
    const int wr = (MODE == 0 && r >= BNW) ? r - BNW : r;
    wsrc[j] = wb + g * gstride + w_offset<bf16_t>(n0 + wr, c * 8, K, blocked);
  }
  const int kw = w_kstep<bf16_t>(blocked);  // weight elements per 64-wide stage of K (BK = 64 = EB)
  int xcnt = 0;  // x DMA instructions this wave issues per stage
#pragma unroll
  for (int j = 0; j < XI; ++j) xcnt += xany[j] ? 1 : 0;
  auto xbuf = [&](int kt) { return lds + (kt % XS) * XBYTES; };
  auto wbuf = [&](int kt) { return lds + XS * XBYTES + (kt % WS) * WBYTES; };
  auto issue_x = [&](int kt) {
    char* sb = xbuf(kt);
    const int ko = kt * BK;
#pragma unroll
    for (int j = 0; j < XI; ++j)
      if (xany[j] && xon[j])
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(xsrc[j] + ko), (lds_ptr_t)(sb + (j * NW + wave) * 1024), 16, 0, 0);
  };
  auto issue_w = [&](int kt, auto nt_c) {
    constexpr int AUX = decltype(nt_c)::value ? 2 : 0;  // 2: non-temporal
    char* sb = wbuf(kt);
#pragma unroll
    for (int j = 0; j < WI; ++j)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wsrc[j] + kt * kw), (lds_ptr_t)(sb + (j * NW + wave) * 1024),
                                       16, 0, AUX);
  };
  const int nk = K / BK;
  auto on = [&](int t) { return t >= 0 && t < nk; };  // t is a stage of K
  // barrier j: x(j + XS), then w(j + WS)
  auto barrier_issue = [&](int j, auto nt_c) {
    if (on(j + XS)) issue_x(j + XS);
    if (on(j + WS)) issue_w(j + WS, nt_c);
  };
  // DMA instructions this wave issued after the later of x(s) and w(s), once
  // the barriers up to s - 2 have issued theirs
  auto after = [&](int s) {
    const int bx = s - XS, bw = s - WS, L = bx > bw ? bx : bw;
    int n = (bx > bw && on(L + WS)) ? WI : 0;  // the same barrier's w, issued after x(s)
#pragma unroll
    for (int q = 1; q <= MINS - 2; ++q) {      // barriers L + 1 .. s - 2
      const int j = L + q;
      n += (on(j + XS) ? xcnt : 0) + (on(j + WS) ? WI : 0);
    }
    return n;
  };
  constexpr int WAITMAX = (MAXS * (XI + WI) < 63) ? MAXS * (XI + WI) : 63;

  f32x16_t acc[NMAT * TNW][TMW];
#pragma unroll
  for (int q = 0; q < NMAT * TNW; ++q)
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[q][i][e] = 0.f;

  // ---- fragments: lane l supplies tile row (l % 32) and K chunk 2s + l/32 of
  // k16 step s (A = weights, B = activations) ----
  const int l32 = lane & 31, lh = lane >> 5;
  // Row tiles of this wave that hold rows of the block (wave-uniform): the
  // MFMAs and fragment reads of the empty 32-row tiles of a partly filled
  // block are skipped (LIVE = 0: the wave only loads and synchronises).
  const int wrows = rows - wm * (BM / WM);
  const int live = wrows <= 0 ? 0 : min(TMW, (wrows + 31) / 32);

  auto main_loop = [&](auto live_c, auto nt_c) {
    constexpr int LIVE = decltype(live_c)::value;
    u32x4_t fw[2][NMAT * TNW], fx[2][TMW > 0 ? TMW : 1];
    auto load_frags = [&](int buf, int s, int slot) {
      if constexpr (LIVE > 0) {
        const char* xs = xbuf(buf);
        const char* ws = wbuf(buf);
#pragma unroll
        for (int i = 0; i < LIVE; ++i)
          fx[slot][i] = *reinterpret_cast<const u32x4_t*>(xs + lds_off(wm * (BM / WM) + i * 32 + l32, 2 * s + lh));
#pragma unroll
        for (int q = 0; q < NMAT * TNW; ++q) {
          const int mat = q / TNW, tj = q % TNW;
          fw[slot][q] = *reinterpret_cast<const u32x4_t*>(
              ws + lds_off(mat * BNW + wn * (BNW / WN) + tj * 32 + l32, 2 * s + lh));
        }
      }
    };
    auto mma = [&](int slot) {
#pragma unroll
      for (int q = 0; q < NMAT * TNW; ++q)
#pragma unroll
        for (int i = 0; i < LIVE; ++i)
          acc[q][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fw[slot][q]),
                                                              __builtin_bit_cast(bf16x8_t, fx[slot][i]), acc[q][i], 0,
                                                              0, 0);
    };
    // one k16 step: the next step's fragment reads alternate with this step's MFMAs
    constexpr int NFRAG = LIVE > 0 ? NMAT * TNW + LIVE : 0, NMMA = NMAT * TNW * LIVE;
    constexpr int NPAIR = NFRAG < NMMA ? NFRAG : NMMA;
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      if constexpr (NMMA > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NPAIR, 0);
      if constexpr (NFRAG > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NFRAG - NPAIR, 0);
    };

#pragma unroll
    for (int j = -MAXS; j < 0; ++j) barrier_issue(j, nt_c);
    // stage 0 landed; what barrier -1 and the ones before it issued after it
    // may still be in flight
    vm_wait_dyn<WAITMAX>(after(0) + (on(XS - 1) ? xcnt : 0) + (on(WS - 1) ? WI : 0));
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    load_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt;  // stage index; the buffers are taken modulo their ring sizes
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) {
          load_frags(buf, s + 1, (s + 1) & 1);
        } else {
          // Stage kt+1 landed (later stages may still be in flight) and this
          // wave's reads of buffer kt are complete: after the barrier the buffer
          // is refilled.  On the last stage nothing is waited for and the reads
          // below touch a buffer whose values are never used, which keeps the
          // step branch-free so its reads interleave with its MFMAs.
          vm_wait_dyn<WAITMAX>(kt + 1 < nk ? after(kt + 1) : 0);
          lgkm_wait0();
          compiler_fence();
          __builtin_amdgcn_s_barrier();
          compiler_fence();
          barrier_issue(kt, nt_c);
          load_frags(kt + 1, 0, 0);
        }
        mma(s & 1);
        interleave();
      }
    }
  };
  auto dispatch = [&](auto self, auto c, auto nt_c) {
    constexpr int L = decltype(c)::value;
    if constexpr (L == 0) {
      main_loop(c, nt_c);
    } else {
      if (live >= L) main_loop(c, nt_c);
      else self(self, std::integral_constant<int, L - 1>{}, nt_c);
    }
  };
  if (NTW && !second)
    dispatch(dispatch, std::integral_constant<int, TMW>{}, std::integral_constant<bool, NTW != 0>{});
  else
    dispatch(dispatch, std::integral_constant<int, TMW>{}, std::false_type{});

  // ---- epilogue: element e of acc[q][i] is D[n = 8*(e/4) + 4*lh + e%4][m = l32]
  // of the 32x32 tile (n: weight row, m: tile row).  A lane holds 4 adjacent
  // columns of a row, so stores straight from the fragments are 8 bytes wide
  // and each store instruction touches 32 rows, 16 bytes of each.
  //   EPI 0: so stored (gate/up only).  Where each expert's weights are
  //     re-read by several row tiles (the layer is compute-bound) this is the
  //     fastest: 464 us against 480 us staged (256 experts x 437..588 rows,
  //     d = 2048, I = 384).
  //   EPI 1, 2: the tile (H, or the down projection's Y) is staged in LDS
  //     (the ring is free now) and leaves row by row in 16-byte chunks, whole
  //     128-byte lines per eight lanes; with EPI 2 as non-temporal stores.
  //     The down projection's d-wide rows always take this path (stored from
  //     the fragments its store stream cost about a quarter of the kernel).
  //     Where the launch streams weights, ordinary stores of H (about 100 MB
  //     against 15 GB of weights in a 256-expert, 7168-wide prefill) slowed
  //     the weight stream of the whole gate/up launch by 7%, and by a fifth
  //     with the MFMAs taken out; the next kernel reads H or Y once, in
  //     another order, so those launches store non-temporally. ----
  static_assert(EPI >= 0 && EPI <= 2 && (MODE == 0 || EPI > 0), "epilogue");
  if constexpr (EPI == 0) {
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const int m = wm * (BM / WM) + i * 32 + l32;
      if (m >= rows) continue;
      bf16_t* orow = out + (size_t)(row0 + m) * N + n0 + wn * (BNW / WN) + 4 * lh;
#pragma unroll
      for (int tj = 0; tj < TNW; ++tj)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x16_t& gt = acc[tj][i];
          const f32x16_t& up = acc[TNW + tj][i];
          const uint32_t o0 = (uint32_t)f32_to_bf16(silu(gt[4 * e4 + 0]) * up[4 * e4 + 0]) |
                              ((uint32_t)f32_to_bf16(silu(gt[4 * e4 + 1]) * up[4 * e4 + 1]) << 16);
          const uint32_t o1 = (uint32_t)f32_to_bf16(silu(gt[4 * e4 + 2]) * up[4 * e4 + 2]) |
                              ((uint32_t)f32_to_bf16(silu(gt[4 * e4 + 3]) * up[4 * e4 + 3]) << 16);
          *reinterpret_cast<uint2*>(orow + tj * 32 + 8 * e4) = make_uint2(o0, o1);
        }
    }
    return;
  }
  vm_wait<0>();
  lgkm_wait0();
  compiler_fence();
  __syncthreads();
  compiler_fence();
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
    const int r = wm * (BM / WM) + i * 32 + l32;
    char* srow = lds + r * EPITCH + (wn * (BNW / WN) + 4 * lh) * 2;
#pragma unroll
    for (int tj = 0; tj < TNW; ++tj)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        uint32_t o0, o1;
        if constexpr (MODE == 0) {
          const f32x16_t& gt = acc[tj][i];
          const f32x16_t& up = acc[TNW + tj][i];
          o0 = (uint32_t)f32_to_bf16(silu(gt[4 * e4 + 0]) * up[4 * e4 + 0]) |
               ((uint32_t)f32_to_bf16(silu(gt[4 * e4 + 1]) * up[4 * e4 + 1]) << 16);
          o1 = (uint32_t)f32_to_bf16(silu(gt[4 * e4 + 2]) * up[4 * e4 + 2]) |
               ((uint32_t)f32_to_bf16(silu(gt[4 * e4 + 3]) * up[4 * e4 + 3]) << 16);
        } else {
          const f32x16_t& y = acc[tj][i];
          o0 = (uint32_t)f32_to_bf16(y[4 * e4 + 0]) | ((uint32_t)f32_to_bf16(y[4 * e4 + 1]) << 16);
          o1 = (uint32_t)f32_to_bf16(y[4 * e4 + 2]) | ((uint32_t)f32_to_bf16(y[4 * e4 + 3]) << 16);
        }
        *reinterpret_cast<uint2*>(srow + (tj * 32 + 8 * e4) * 2) = make_uint2(o0, o1);
      }
  }
  __syncthreads();
  constexpr int CPR = BNW * 2 / 16;  // 16-byte chunks per row
  const int live_rows = min(BM, rows);
  for (int q = tid; q < live_rows * CPR; q += 64 * NW) {
    const int r = q / CPR, ch = q - r * CPR;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + r * EPITCH + ch * 16);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + r) * N + n0 + ch * 8);
    if constexpr (EPI == 2) __builtin_nontemporal_store(v, dst);
    else *dst = v;
  }
}

// Tile height of the configuration launch_ffn_*_gemm picks for rows_hint, which
// is also the row-block height of the tile table.
int gemm_row_block(int rows_hint) { return rows_hint >= 256 ? 256 : 128; }

template <int MODE, int BM, int BNW, int WM, int WN, int XS, int WS, int NTW = 0, int EPI = 1>
static hipError_t launch_gemm_variant(const void* in, const int32_t* row_map, const void* w0, const void* w1,
                                      const int4* blocks, int bound, int dense_rows, void* out, int N, int K,
                                      int blocked, hipStream_t st, const GemmSecond& sec = GemmSecond{}) {
  if (N % BNW != 0 || K % BK != 0) return hipErrorInvalidValue;
  const int rb_bound = blocks ? bound : (dense_rows + BM - 1) / BM;
  const long long total = ((long long)rb_bound + (sec.rows + BM - 1) / BM) * (N / BNW);
  if (total == 0) return hipSuccess;
  // eight XCD ranges, each a whole share of both problems' tiles (the kernel's mapping)
  const long long nwg = 8 * ((rb_bound * (N / BNW) + 7) / 8 + ((long long)((sec.rows + BM - 1) / BM) * (N / BNW) + 7) / 8);
  if (nwg > 0x7fffffffLL / (64 * WM * WN)) return hipErrorInvalidValue;
  if (sec.rows > 0)
    hipLaunchKernelGGL((ffn_gemm_kernel<MODE, BM, BNW, WM, WN, XS, WS, NTW, EPI, true>), dim3((unsigned)nwg),
                       dim3(64 * WM * WN), 0, st, (const bf16_t*)in, row_map, (const bf16_t*)w0, (const bf16_t*)w1,
                       blocks, bound, dense_rows, (bf16_t*)out, N, K, (const bf16_t*)sec.in, (const bf16_t*)sec.w0,
                       (const bf16_t*)sec.w1, (bf16_t*)sec.out, sec.rows, blocked);
  else
    hipLaunchKernelGGL((ffn_gemm_kernel<MODE, BM, BNW, WM, WN, XS, WS, NTW, EPI, false>), dim3((unsigned)nwg),
                       dim3(64 * WM * WN), 0, st, (const bf16_t*)in, row_map, (const bf16_t*)w0, (const bf16_t*)w1,
                       blocks, bound, dense_rows, (bf16_t*)out, N, K, nullptr, nullptr, nullptr, nullptr, 0,
                       blocked);
  return hipGetLastError();
}

// Tile height: 256-row tiles when groups hold hundreds of rows (fewer weight
// re-reads per flop); 128-row tiles when they hold about a hundred, where a
// 256-row tile would be mostly empty (there the layer streams weights).
// Measured with flushed caches (256 experts x 96 rows, d = 7168, I = 2048;
// 256 experts x 437..588 rows, d = 2048, I = 384):
//  - the 128-row tiles stream weights.  Gate/up: non-temporal weight DMA and
//    output stores, and 256 columns per tile where I allows (2452 us; 2540
//    with 128 columns and a 3-deep ring, 2650 with neither hint): each
//    gathered activation stage then feeds twice the weights, and those
//    activation loads were the costliest part of the launch (2313 us without
//    them).  Down: non-temporal stores alone (1520 with the weight hint as
//    well), 8 waves and 512 columns where d allows (1388 us; 1424 with 256
//    columns, 1493 with 256 columns and 4 waves).
//  - the 256-row tiles re-read each expert's weights from the cache and keep
//    ordinary loads and stores (gate/up 454 and down 373 us in the layer, 470
//    and 384 with both hints).
hipError_t launch_ffn_gateup_gemm(const void* in, const int32_t* row_map, const void* wg, const void* wu,
                                  const int4* blocks, int bound, int dense_rows, int rows_hint, void* h, int N,
                                  int K, int blocked, hipStream_t st, const GemmSecond& sec) {
  if (gemm_row_block(rows_hint) == 256)
    return launch_gemm_variant<0, 256, 128, 4, 2, 2, 3, 0, 0>(in, row_map, wg, wu, blocks, bound, dense_rows, h, N, K,
                                                              blocked, st, sec);
  if (N % 256 == 0)
    return launch_gemm_variant<0, 128, 256, 2, 4, 2, 2, 1, 2>(in, row_map, wg, wu, blocks, bound, dense_rows, h, N, K,
                                                              blocked, st, sec);
  return launch_gemm_variant<0, 128, 128, 2, 4, 3, 3, 1, 2>(in, row_map, wg, wu, blocks, bound, dense_rows, h, N, K,
                                                            blocked, st, sec);
}

hipError_t launch_ffn_down_gemm(const void* h, const int32_t* row_map, const void* wd, const int4* blocks, int bound,
                                int dense_rows, int rows_hint, void* y, int N, int K, int blocked, hipStream_t st,
                                const GemmSecond& sec) {
  if (gemm_row_block(rows_hint) == 256) {
    if (N % 256 == 0)
      return launch_gemm_variant<1, 256, 256, 4, 2, 2, 3>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K,
                                                          blocked, st, sec);
    return launch_gemm_variant<1, 256, 128, 4, 2, 2, 3>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K, blocked,
                                                        st, sec);
  }
  if (N % 512 == 0)
    return launch_gemm_variant<1, 128, 512, 2, 4, 2, 2, 0, 2>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K,
                                                              blocked, st, sec);
  if (N % 256 == 0)
    return launch_gemm_variant<1, 128, 256, 2, 4, 2, 3, 0, 2>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K,
                                                              blocked, st, sec);
  return launch_gemm_variant<1, 128, 128, 2, 2, 3, 3, 0, 2>(h, row_map, wd, wd, blocks, bound, dense_rows, y, N, K,
                                                            blocked, st, sec);
}

}  // namespace moe
