// probe.hip -- a plain HBM read, to measure what the part streams.
//
// Not a step of the method: the score kernel's HBM rate is judged against
// this, the rate at which the same part reads the same bytes with nothing
// else to do.  The units (pages) are shared out the way the score kernel
// shares its pages: every workgroup of a resident grid takes an equal
// contiguous share of the unit list, and streams it with 16-byte loads, 16
// loads a thread in flight.  Each unit is at least 1 KB, so the 64 pieces a
// wave loads at once lie in one unit and the unit's id is a scalar load.
#include <atomic>

#include "device.h"

namespace idx {

constexpr int kProbeThreads = 512;
constexpr int kProbeLoads = 16;  // 16-byte loads a thread keeps in flight

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* base, int64_t n_base_units,
                                                                   const int32_t* units, int64_t n_units,
                                                                   int ppu_shift, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t lo = (int64_t)blockIdx.x * n_units / gridDim.x;
  const int64_t hi = (int64_t)(blockIdx.x + 1) * n_units / gridDim.x;
  const int64_t p_hi = hi << ppu_shift;  // pieces of 16 bytes
  const int64_t ppu_mask = ((int64_t)1 << ppu_shift) - 1;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (int64_t p0 = lo << ppu_shift; p0 < p_hi; p0 += kProbeLoads * kProbeThreads) {
    u32x4 v[kProbeLoads];
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) {
      const int64_t pw = p0 + (int64_t)kProbeThreads * k + 64 * wave;  // the wave's first piece
      v[k] = u32x4{0u, 0u, 0u, 0u};
      if (pw < p_hi) {  // wave-uniform: shares end on unit bounds, units hold >= 64 pieces
        const int64_t u = pw >> ppu_shift;
        int64_t id = units ? (int64_t)units[u] : u;
        if (id < 0 || id >= n_base_units) id = 0;
        const u32x4* src = base + (id << ppu_shift) + (pw & ppu_mask) + lane;
        v[k] = NT ? __builtin_nontemporal_load(src) : *src;
      }
    }
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) acc ^= v[k];
  }
  // one word a workgroup, so that no load can be dropped
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int d = 32; d >= 1; d >>= 1) x ^= __shfl_xor(x, d);
  __shared__ uint32_t red[kProbeThreads / 64];
  if (lane == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

namespace {
template <bool NT>
int probe_grid() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int n = cache[dev].load(std::memory_order_relaxed); n > 0) return n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(read_probe_kernel<NT>),
                                                   kProbeThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev].store(cus * per_cu, std::memory_order_relaxed);
  return cus * per_cu;
}
}  // namespace

hipError_t launch_read_probe(const void* base, int64_t n_base_units, const int32_t* units, int64_t n_units,
                             int unit_bytes, bool nt, uint32_t* sink, int n_sink, hipStream_t stream) {
  if (n_units == 0) return hipSuccess;
  const int ppu_shift = __builtin_ctz((unsigned)unit_bytes) - 4;
  const int grid = min(n_sink, nt ? probe_grid<true>() : probe_grid<false>());
  if (nt)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(base), n_base_units, units, n_units, ppu_shift, sink);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(base), n_base_units, units, n_units, ppu_shift, sink);
  return hipGetLastError();
}

}  // namespace idx
