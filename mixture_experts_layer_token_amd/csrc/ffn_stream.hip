// Weight-streaming grouped SwiGLU FFN on MFMA (the memory-bound decode path).
//
// In decode the layer's time is the time to load the activated experts'
// weights from HBM (METRO reading notes, arXiv 2512.09277, Q1; ExFold summary,
// arXiv 2608.24938, MoE Inference: decode is batch-memory bound), so every
// weight byte is read exactly once, with 16-byte loads, by one wave, while the
// few rows routed to that expert ride along on the narrow side of a 16x16 MFMA.
//
// Work split.  Grid = (column tiles, groups).  A workgroup is 4 waves = WN
// waves along the output columns x WK waves along K.  A wave owns two 16-row
// weight tiles:
//   gate/up: rows c..c+15 of W_gate and of W_up (same 16 output columns)
//   down:    rows c..c+31 of W_down (two 16-column tiles)
// and for each K step loads, per lane, KC contiguous elements of one weight
// row per tile (lane l: row l%16, K offset (l/16)*KC).  The activation rows use
// the same K indices on the other MFMA side, so the instruction sums exactly
// the K values the lanes supplied (any consistent K order gives the dot
// product).  Rows are processed 64 at a time (4 MFMA column tiles); waves along
// K add their partial sums through LDS in a fixed order.
//
// The gate/up epilogue applies SwiGLU (MoE-Prism, arXiv 2510.19366, §III-B1,
// Eq. (1)): H = SiLU(g) * u, stored in the element type.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int SMT = 4;  // MFMA column tiles (16 rows each) per row group

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

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// MODE 0: gate/up + SwiGLU.  MODE 1: down projection.
template <typename T, int MODE, int KC, int WK>
__global__ __launch_bounds__(256) void ffn_stream_kernel(const T* __restrict__ in,
                                                         const int32_t* __restrict__ row_map,
                                                         const T* __restrict__ w0, const T* __restrict__ w1,
                                                         const int32_t* __restrict__ grp_off, int dense_rows,
                                                         T* __restrict__ out, int N, int K) {
  constexpr int WN = 4 / WK;
  constexpr int CPW = (MODE == 0) ? 16 : 32;  // output columns per wave
  constexpr int NB = WN * CPW;                // output columns per workgroup
  constexpr int LE = 16 / sizeof(T);          // elements per 16-byte load
  constexpr int LPS = KC / LE;                // loads per tile row per K step
  static_assert(KC % LE == 0, "K step must be whole 16-byte loads");
  __shared__ f32x4_t red[(WK > 1) ? (WK - 1) * WN * SMT * 2 * 64 : 1];

  const int g = blockIdx.y;
  int row0, rows;
  if (grp_off) {
    row0 = grp_off[g];
    rows = grp_off[g + 1] - row0;
  } else {
    row0 = 0;
    rows = dense_rows;
  }
  if (rows <= 0) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % WN, wk = wave / WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * NB + wn * CPW;
  const int Kw = K / WK;
  const int kbeg = wk * Kw, kend = kbeg + Kw;
  const size_t gstride = (size_t)N * K;
  const T* wa;
  const T* wb;
  if (MODE == 0) {
    wa = w0 + g * gstride + (size_t)(n0 + lr) * K;
    wb = w1 + g * gstride + (size_t)(n0 + lr) * K;
  } else {
    wa = w0 + g * gstride + (size_t)(n0 + lr) * K;
    wb = w0 + g * gstride + (size_t)(n0 + 16 + lr) * K;
  }

  for (int mg = 0; mg < rows; mg += 16 * SMT) {
    const int mts = min(SMT, (rows - mg + 15) >> 4);  // live column tiles (wave-uniform)
    const T* xr[SMT];
    bool valid[SMT];
#pragma unroll
    for (int mt = 0; mt < SMT; ++mt) {
      const int r = mg + mt * 16 + lr;
      valid[mt] = r < rows;
      const int src = valid[mt] ? (row_map ? row_map[row0 + r] : row0 + r) : 0;
      xr[mt] = in + (size_t)src * K;
    }
    f32x4_t acc[SMT][2];
#pragma unroll
    for (int mt = 0; mt < SMT; ++mt) {
      acc[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    for (int kc = kbeg; kc < kend; kc += 4 * KC) {
      const int ko = kc + lg * KC;
      uint4 A0[LPS], A1[LPS];
#pragma unroll
      for (int i = 0; i < LPS; ++i) {
        A0[i] = ld16(wa + ko + i * LE);
        A1[i] = ld16(wb + ko + i * LE);
      }
#pragma unroll
      for (int mt = 0; mt < SMT; ++mt) {
        if (mt < mts) {
          uint4 B[LPS];
#pragma unroll
          for (int i = 0; i < LPS; ++i) B[i] = valid[mt] ? ld16(xr[mt] + ko + i * LE) : zero_u4();
#pragma unroll
          for (int i = 0; i < LPS; ++i) {
            mma_tile<T>(acc[mt][0], A0[i], B[i]);
            mma_tile<T>(acc[mt][1], A1[i], B[i]);
          }
        }
      }
    }

    if (WK > 1) {
      if (wk > 0) {
#pragma unroll
        for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            red[((((wk - 1) * WN + wn) * SMT + mt) * 2 + tt) * 64 + lane] = acc[mt][tt];
      }
      __syncthreads();
      if (wk == 0) {
        for (int q = 1; q < WK; ++q) {
#pragma unroll
          for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[mt][tt] += red[((((q - 1) * WN + wn) * SMT + mt) * 2 + tt) * 64 + lane];
        }
      }
    }

    if (wk == 0) {
#pragma unroll
      for (int mt = 0; mt < SMT; ++mt) {
        const int m = mg + mt * 16 + lr;
        if (mt < mts && m < rows) {
          T* orow = out + (size_t)(row0 + m) * N;
          if (MODE == 0) {
            const f32x4_t gt = acc[mt][0], up = acc[mt][1];
            store4<T>(orow + n0 + 4 * lg, silu(gt[0]) * up[0], silu(gt[1]) * up[1], silu(gt[2]) * up[2],
                      silu(gt[3]) * up[3]);
          } else {
            const f32x4_t y0 = acc[mt][0], y1 = acc[mt][1];
            store4<T>(orow + n0 + 4 * lg, y0[0], y0[1], y0[2], y0[3]);
            store4<T>(orow + n0 + 16 + 4 * lg, y1[0], y1[1], y1[2], y1[3]);
          }
        }
      }
    }
    if (WK > 1) __syncthreads();
  }
}

template <typename T, int MODE, int KC, int WK>
static hipError_t launch_one(const T* in, const int32_t* row_map, const T* w0, const T* w1, const int32_t* grp_off,
                             int G, int dense_rows, T* out, int N, int K, hipStream_t st) {
  constexpr int NB = (4 / WK) * ((MODE == 0) ? 16 : 32);
  dim3 grid(N / NB, G);
  hipLaunchKernelGGL((ffn_stream_kernel<T, MODE, KC, WK>), grid, dim3(256), 0, st, in, row_map, w0, w1, grp_off,
                     dense_rows, out, N, K);
  return hipGetLastError();
}

// K split across the workgroup's waves for the down projection: long K and few
// output columns per expert want more waves along K.
static int pick_wk(int K, int step) {
  if (K >= 4096 && K % (4 * step) == 0) return 4;
  if (K >= 512 && K % (2 * step) == 0) return 2;
  return 1;
}

template <typename T>
static hipError_t gateup_t(const void* in, const int32_t* row_map, const void* wg, const void* wu,
                           const int32_t* grp_off, int G, int dense_rows, void* h, int N, int K, hipStream_t st) {
  constexpr int KC = (sizeof(T) == 2) ? 32 : 8;
  return launch_one<T, 0, KC, 1>((const T*)in, row_map, (const T*)wg, (const T*)wu, grp_off, G, dense_rows, (T*)h,
                                 N, K, st);
}

template <typename T>
static hipError_t down_t(const void* h, const void* wd, const int32_t* grp_off, int G, int dense_rows, void* y,
                         int N, int K, hipStream_t st) {
  constexpr int KC = (sizeof(T) == 2) ? 32 : 8;
  const int wk = pick_wk(K, 4 * KC);
  const T* in = (const T*)h;
  const T* w = (const T*)wd;
  T* out = (T*)y;
  if (wk == 4) return launch_one<T, 1, KC, 4>(in, nullptr, w, w, grp_off, G, dense_rows, out, N, K, st);
  if (wk == 2) return launch_one<T, 1, KC, 2>(in, nullptr, w, w, grp_off, G, dense_rows, out, N, K, st);
  return launch_one<T, 1, KC, 1>(in, nullptr, w, w, grp_off, G, dense_rows, out, N, K, st);
}

hipError_t launch_ffn_gateup_stream(int dtype, const void* in, const int32_t* row_map, const void* wg,
                                    const void* wu, const int32_t* grp_off, int G, int dense_rows, void* h,
                                    int N, int K, hipStream_t st) {
  if (dtype == DT_BF16) return gateup_t<bf16_t>(in, row_map, wg, wu, grp_off, G, dense_rows, h, N, K, st);
  return gateup_t<float>(in, row_map, wg, wu, grp_off, G, dense_rows, h, N, K, st);
}

hipError_t launch_ffn_down_stream(int dtype, const void* h, const void* wd, const int32_t* grp_off, int G,
                                  int dense_rows, void* y, int N, int K, hipStream_t st) {
  if (dtype == DT_BF16) return down_t<bf16_t>(h, wd, grp_off, G, dense_rows, y, N, K, st);
  return down_t<float>(h, wd, grp_off, G, dense_rows, y, N, K, st);
}

}  // namespace moe
