// moe_forward_noalloc: moe_forward with its scratch in a library-held device
// array instead of a caller workspace, for callers that cannot allocate
// device memory (code under HIP-graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The array `scratch` below is a file-scope __device__ variable: every GPU
// the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the name `scratch` is only a host-side handle
// of that variable, not a device address, so it is never passed to a kernel
// or a copy; the device address is looked up once per device (with that
// device current) by hipGetSymbolAddress, kept in `g_scratch`, and that
// pointer is what the kernels receive.
//
// The forward's kernels write every scratch region before they read it
// (routing arrays, partial sums, the row-block table, H, Y), so nothing in
// the array needs clearing between calls.  Calls on one GPU share that GPU's
// array: two calls that overlap in time on one device (two streams, two host
// threads) race on it.
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first
// call on the device.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                                          const float* router_bias, const int32_t* k, const void* w_gate,
                                          const void* w_up, const void* w_down, const void* ws_gate,
                                          const void* ws_up, const void* ws_down, void* out, int32_t* stats,
                                          int32_t* dev_status, moe_stream_t stream) {
  // the descriptor and the size are checked before anything touches the device
  moe_status s = moe::forward_scratch_check(desc, kScratchBytes);
  if (s != MOE_OK) return s;
  void* p = nullptr;
  s = scratch_ptr(&p);
  if (s != MOE_OK) return s;
  return moe::forward_impl(desc, x, w_router, router_bias, k, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out,
                           stats, dev_status, p, kScratchBytes, stream, true);
}
