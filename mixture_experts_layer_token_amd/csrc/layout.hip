// Row-major -> blocked copy of a stack of expert weight matrices.
//
// The blocked order (w_offset in common.h) stores each [N][K] matrix as
// 64-row x 128-byte blocks, so the 64 rows x 128 bytes that a streaming or
// GEMM workgroup reads per step of K are one contiguous 8 KB run instead of 64
// lines one matrix row apart.  The copy runs once per weight stack, when it
// is loaded.  One thread per 16-byte chunk: a source row is read contiguously
// and each group of eight threads writes one whole 128-byte row of a block.
#include "common.h"
#include "launch.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void pack_weights_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                           long long chunks, int N, int K) {
  constexpr int LE = 16 / sizeof(T);
  const int cpr = K / LE;  // chunks per row
  for (long long q = blockIdx.x * 256ll + threadIdx.x; q < chunks; q += (long long)gridDim.x * 256) {
    const long long row = q / cpr;  // row of the whole stack
    const int k = (int)(q - row * cpr) * LE;
    const long long g = row / N;
    const int n = (int)(row - g * N);
    const size_t base = (size_t)g * N * K;
    *reinterpret_cast<uint4*>(dst + base + w_offset<T>(n, k, K, 1)) =
        *reinterpret_cast<const uint4*>(src + base + (size_t)n * K + k);
  }
}

hipError_t launch_pack_weights(int dtype, long long G, int N, int K, const void* src, void* dst, hipStream_t st) {
  const int le = dtype == DT_BF16 ? 8 : 4;
  const long long chunks = G * N * (long long)(K / le);
  if (chunks == 0) return hipSuccess;
  const long long want = (chunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(pack_weights_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)src, (bf16_t*)dst,
                       chunks, N, K);
  else
    hipLaunchKernelGGL(pack_weights_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)src, (float*)dst,
                       chunks, N, K);
  return hipGetLastError();
}

}  // namespace moe
