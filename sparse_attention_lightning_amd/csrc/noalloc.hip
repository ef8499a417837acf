// noalloc.hip -- idx_step for callers that cannot allocate device memory.
//
// idx_step hands the block scores from the score kernel to the top-k kernel
// through a caller-owned buffer.  idx_step_noalloc keeps that hand-off in a
// file-scope device array instead, so its caller passes only the step's
// inputs and its top-k outputs, and the call allocates nothing.  Each device
// holds its own copy of the array (16 MiB) until the process ends.  Host
// code never passes the array's name to a kernel: on the host that name is a
// stand-in, not a device address.  Its address on each device is looked up
// once, with that device current, and kept per device.
#include <mutex>

#include "device.h"

// The block-score hand-off of idx_step_noalloc, every device its own copy.
static __device__ __align__(256) float scratch[IDX_NOALLOC_MAX_SCORES];

namespace idx {
namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
float* g_ptr[kMaxDevices];  // the array's device address per device (under g_mu)

}  // namespace

hipError_t noalloc_scores(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace idx
