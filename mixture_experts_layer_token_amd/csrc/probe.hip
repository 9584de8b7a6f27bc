// Streaming-read probe: the HBM read rate a plain kernel reaches on this part,
// printed beside the layer's roofline figures as the practical ceiling of a
// weight stream (the nominal 8 TB/s is not reachable by reads alone).  Not a
// step of the layer.
//
// Each workgroup step reads UNROLL contiguous 4 KB runs (256 threads x 16
// bytes each), all in flight at once; workgroups take steps round-robin over
// the buffer, two workgroups per CU.  Of a sweep over run length, loads in
// flight (4 to 16 per thread), round-robin runs or one contiguous window per
// workgroup, and 2 to 8 workgroups per CU over 4 GiB, this read fastest with
// the non-temporal hint (7.1-7.3 TB/s; ordinary loads 6.0-6.3 TB/s).
// The loaded words are folded into one value per thread, which is stored only
// if it equals a constant that a fold of real data practically never hits, so
// the loads cannot be dropped.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {
constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 4;
constexpr int PROBE_WG_PER_CU = 2;
}  // namespace

template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t run = (size_t)PROBE_THREADS * PROBE_UNROLL;  // 16-byte items per workgroup step
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * run; base < n16; base += (size_t)gridDim.x * run) {
    uint4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) {
      const size_t i = base + (size_t)u * PROBE_THREADS + threadIdx.x;
      if (i < n16) {
        if (NT) {
          const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i));
          v[u] = make_uint4(t[0], t[1], t[2], t[3]);
        } else {
          v[u] = src[i];
        }
      } else {
        v[u] = zero_u4();
      }
    }
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, int nontemporal, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t run = (size_t)PROBE_THREADS * PROBE_UNROLL;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const size_t steps = (n16 + run - 1) / run;
  const size_t want = (size_t)cus * PROBE_WG_PER_CU;
  const unsigned grid = (unsigned)(steps < want ? steps : want);
  if (nontemporal)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(grid), dim3(PROBE_THREADS), 0, st, (const uint4*)src, n16, sink);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(grid), dim3(PROBE_THREADS), 0, st, (const uint4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace moe
