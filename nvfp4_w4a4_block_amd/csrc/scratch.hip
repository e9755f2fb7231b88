// Fixed device scratch for callers that cannot allocate: the workspace of the
// split-K M-tile GEMM (arrival counters, then fp32 partial sums) held in a
// file-scope device array instead of a caller buffer.
//
// The array's name is a host-side stand-in in host code, not a device
// address: the address of each device's copy is taken once per device with
// hipGetSymbolAddress (with that device current) and kept; only that address
// is ever passed to a kernel.  At the same set-up the counter area is cleared
// by a small fill kernel on the caller's stream (stream-ordered, and valid
// under graph capture, where a memset node is not used); every call leaves
// the counters zero again.
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
constexpr uint32_t kCounterBytes = 64 * 1024;  // covers the arrival counters of any split plan

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = threadIdx.x + blockIdx.x * blockDim.x; i < n; i += blockDim.x * gridDim.x) p[i] = 0u;
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_workspace(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    clear_words_kernel<<<16, 256, 0, stream>>>(static_cast<uint32_t*>(p), kCounterBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nvfp4
