// topk.hip -- forced block top-k per (row, head) for gfx950.
//
// Selection (sglang PR 42614, Modifications item 1 and Accuracy Tests): with
// nb = ceil(row_len / 128) blocks, every block is taken when nb <= topk;
// otherwise the first init_blocks and the last local_blocks of the row's own
// nb are always taken and the remaining slots go to the highest block scores,
// ties to the lower block id.  Selection is exact.
//
// One workgroup per (row, head).  Each block gets a 32-bit key whose unsigned
// order is the selection order: forced blocks get the largest key, scores map
// to an order-preserving integer (NaN below every number, -0 equal to +0).
// An MSB-first radix select (4 passes of 8 bits, LDS histograms) finds the
// topk-th largest key T and how many keys equal to T are still needed; one
// ascending pass then emits every key > T and the lowest ids with key == T,
// so ids come out in ascending order without a sort.
#include "device.h"

namespace idx {

constexpr int kTopkThreads = 256;
constexpr uint32_t kForcedKey = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;  // NaN
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 256 threads of the workgroup.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += wave_tot[w];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const StepArgs a) {
  extern __shared__ uint32_t keys[];  // max_blocks entries
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kTopkThreads / 64];
  __shared__ uint32_t pick_digit, pick_above;
  __shared__ uint32_t chunk_tot[2];

  const int tid = threadIdx.x;
  const int rows = a.P * a.H;
  const int o = blockIdx.x;
  const int r = o / rows, i = o - r * rows;
  const int K = a.topk, MB = a.max_blocks;
  int32_t* ids = a.topk_ids + (int64_t)o * K;
  float* sc = a.topk_scores + (int64_t)o * K;
  const float* bs = a.block_scores + (int64_t)o * MB;

  const int slot = a.req_slot[r];
  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  const int nb = pad ? 0 : blocks_of(clamp_len(a.row_len[r * a.P + i / a.H], MB));

  if (nb <= K) {
    for (int t = tid; t < K; t += kTopkThreads) {
      ids[t] = t < nb ? t : -1;
      sc[t] = t < nb ? bs[t] : -INFINITY;
    }
    return;
  }

  const int init = a.init_blocks, local_from = nb - a.local_blocks;
  for (int b = tid; b < nb; b += kTopkThreads)
    keys[b] = (b < init || b >= local_from) ? kForcedKey : order_key(bs[b]);
  __syncthreads();

  // radix select of the K-th largest key
  uint32_t prefix = 0;
  uint32_t want = (uint32_t)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    const uint32_t hi_mask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int b = tid; b < nb; b += kTopkThreads) {
      const uint32_t k = keys[b];
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t looks at digit 255 - t: counts of larger digits come first
    const uint32_t h = hist[255 - tid];
    const uint32_t incl = block_inclusive_scan(h, wave_tot);
    const uint32_t excl = incl - h;
    if (excl < want && want <= incl) {
      pick_digit = 255u - (uint32_t)tid;
      pick_above = excl;
    }
    __syncthreads();
    prefix |= pick_digit << shift;
    want -= pick_above;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // emit in ascending id order: all keys > T, then the first `want` keys == T
  uint32_t out_pos = 0, ties_seen = 0;
  for (int base = 0; base < nb; base += kTopkThreads) {
    const int b = base + tid;
    const uint32_t k = (b < nb) ? keys[b] : 0u;
    const uint32_t gt = (b < nb && k > T) ? 1u : 0u;
    const uint32_t eq = (b < nb && k == T) ? 1u : 0u;
    const uint32_t eq_incl = block_inclusive_scan(eq, wave_tot);
    const uint32_t take = (gt || (eq && ties_seen + eq_incl - 1u < want)) ? 1u : 0u;
    const uint32_t take_incl = block_inclusive_scan(take, wave_tot);
    const uint32_t pos = out_pos + take_incl - 1u;
    if (take && pos < (uint32_t)K) {
      ids[pos] = b;
      sc[pos] = bs[b];
    }
    // totals of this chunk: the last thread's inclusive sums
    if (tid == kTopkThreads - 1) {
      chunk_tot[0] = take_incl;
      chunk_tot[1] = eq_incl;
    }
    __syncthreads();
    out_pos += chunk_tot[0];
    ties_seen += chunk_tot[1];
    __syncthreads();
  }
}

hipError_t launch_topk(const StepArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_req * a.P * a.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t smem = (size_t)(a.max_blocks > 0 ? a.max_blocks : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)grid), dim3(kTopkThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace idx
