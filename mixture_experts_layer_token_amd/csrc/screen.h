// Exact dot products for the screened routers (the MoE router and the
// compositional-path router): a token row against a list of weight rows under
// the routing contract -- products of bf16 values are exact in float32 and in
// float64, the sums are taken in float64 -- one wave per token.
#pragma once

#include "common.h"

namespace moe {

// Summation depth n of the screening pass's float32 sums (the MFMA pass of
// route_screen.hip, which both screened routers use): K is cut into S slices
// of whole 64-element stages, each slice sums its products in float32 in
// whatever order the MFMA adds them, and the S slice sums are added in
// float32: n <= the longest slice's products + S.  The error of such a sum is
// at most n * u * sum |x_i w_i| (u the float32 unit roundoff).
__device__ __forceinline__ double screen_depth(int d, int S) {
  const int chunks = d / 64;
  return (double)(((chunks + S - 1) / S) * 64 + S);
}

// Lane share of an exact dot product over one 8-element chunk: the products
// of bf16 values are exact in float32, each is widened and added in float64.
// acc[q] takes elements 2q and 2q+1 (four independent chains).
__device__ __forceinline__ void dot8(const uint4& xv, const uint4& wv, double (&acc)[4]) {
  const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float p0 = __uint_as_float(xs[q] << 16) * __uint_as_float(ws[q] << 16);
    const float p1 = __uint_as_float(xs[q] & 0xffff0000u) * __uint_as_float(ws[q] & 0xffff0000u);
    acc[q] += (double)p0;
    acc[q] += (double)p1;
  }
}

// The same with the token's eight elements already widened to float64: one
// fused multiply-add per element (the product of two bf16 values is exact in
// float64, so fma(x, w, acc) rounds exactly as acc + x*w does above).
__device__ __forceinline__ void dot8_wide(const double (&xd)[8], const uint4& wv, double (&acc)[4]) {
  const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[q] = fma(xd[2 * q], (double)__uint_as_float(ws[q] << 16), acc[q]);
    acc[q] = fma(xd[2 * q + 1], (double)__uint_as_float(ws[q] & 0xffff0000u), acc[q]);
  }
}

// Exact dot products run in passes of 512 * XC elements (lane l takes
// elements [8l + 512 i, +8) of chunk i).
constexpr int SEL_GRP = 8;  // rows whose cross-lane sums are done together

// Exact dot products of the token row xrow with n rows (row_of(c), c < n),
// under the routing contract: exact products, float64 accumulation.  Work
// items (row c, pass p) in order, p fastest; the rows' chunks of items
// i+1 .. i+DEPTH-1 are requested before item i is summed.  Each lane's share
// of a row goes to red[c % GRP][lane] (GRP * 64 doubles of LDS); every GRP
// rows, lane j adds the 64 shares of row j of the group in lane order and
// calls sink(c, sum).  One wave; ends with the wave's LDS writes visible.
// XR: the token row stays in registers for all rows, widened to float64, or
// with XB as its bf16 words (a quarter of the registers; dot8 then forms the
// same exact products and adds them in the same order, so the sums are the
// same bits).
template <int XC, bool XR, int GRP, int DEPTH = 2, bool XB = false, class RowOf, class Sink>
__device__ __forceinline__ void exact_dots(const bf16_t* __restrict__ xrow, int d, int n, RowOf row_of, double* red,
                                           Sink sink) {
  const int lane = threadIdx.x & 63;
  constexpr int PASS = 512 * XC;
  const int npass = (d + PASS - 1) / PASS;
  const int items = n * npass;
  // resident token row (XR): as bf16 words (XB) or widened to float64 once
  uint4 xb[XR && XB ? XC : 1];
  double xd[XR && !XB ? XC : 1][8];
  if constexpr (XR && XB) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int off = 512 * i + 8 * lane;
      xb[i] = off < d ? *reinterpret_cast<const uint4*>(xrow + off) : zero_u4();
    }
  } else if constexpr (XR) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int off = 512 * i + 8 * lane;
      const uint4 v = off < d ? *reinterpret_cast<const uint4*>(xrow + off) : zero_u4();
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xd[i][2 * q] = (double)__uint_as_float(u[q] << 16);
        xd[i][2 * q + 1] = (double)__uint_as_float(u[q] & 0xffff0000u);
      }
    }
  }
  auto load_item = [&](uint4 (&xv)[XC], uint4 (&wr)[XC], int it) {
    const int c = it / npass, p0 = (it - c * npass) * PASS;
    const bf16_t* row = row_of(c);
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int off = p0 + 512 * i + 8 * lane;
      if constexpr (!XR) xv[i] = off < d ? *reinterpret_cast<const uint4*>(xrow + off) : zero_u4();
      wr[i] = off < d ? *reinterpret_cast<const uint4*>(row + off) : zero_u4();
    }
  };
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  auto finish_item = [&](int it, const uint4 (&xv)[XC], const uint4 (&wr)[XC]) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      if constexpr (XR && XB) dot8(xb[i], wr[i], acc);
      else if constexpr (XR) dot8_wide(xd[i], wr[i], acc);
      else dot8(xv[i], wr[i], acc);
    }
    const int c = it / npass;
    if (it - c * npass == npass - 1) {  // row complete
      red[(c % GRP) * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      acc[0] = acc[1] = acc[2] = acc[3] = 0.0;
      if (c % GRP == GRP - 1 || c == n - 1) {
        const int g0 = c - c % GRP;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane <= c - g0) {
          double v = 0.0;
          for (int l = 0; l < 64; ++l) v += red[lane * 64 + l];
          sink(g0 + lane, v);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  };
  // a register ring of DEPTH items, indexed by compile-time positions
  static_assert(DEPTH >= 2 && DEPTH <= 8, "pipeline depth");
  uint4 xq[DEPTH][XC], wq[DEPTH][XC];
#pragma unroll
  for (int q = 0; q < DEPTH - 1; ++q)
    if (q < items) load_item(xq[q], wq[q], q);
  for (int it = 0; it < items; it += DEPTH) {
#pragma unroll
    for (int q = 0; q < DEPTH; ++q) {
      const int i = it + q;
      if (i + DEPTH - 1 < items) load_item(xq[(q + DEPTH - 1) % DEPTH], wq[(q + DEPTH - 1) % DEPTH], i + DEPTH - 1);
      if (i < items) finish_item(i, xq[q], wq[q]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace moe
