// topk.hip -- forced block top-k per (row, head) for gfx950.
//
// Selection (sglang PR 42614, Modifications item 1 and Accuracy Tests): with
// nb = ceil(row_len / 128) blocks, every block is taken when nb <= topk;
// otherwise the first init_blocks and the last local_blocks of the row's own
// nb are always taken and the remaining topk - |forced| slots go to the
// highest block scores, ties to the lower block id.  Selection is exact.
//
// One workgroup of 256 threads per (row, head).  Thread t owns the contiguous
// blocks [t*C, t*C + C), C = ceil(nb / 256) <= 32, and keeps their scores and
// 32-bit order keys in registers (all loads issued at once).  The key's
// unsigned order is the selection order: NaN below every number, -0 equal to
// +0.  A radix select over the non-forced keys finds the k-th largest key T,
// k = topk - |forced|: it starts at the highest bit where the row's keys
// differ, takes up to 8 bits a pass with an LDS histogram, and stops early
// once the chosen bin holds exactly the keys still needed.  One packed scan of
// (taken-for-sure, equal-to-T) counts then gives every thread its output
// position, so ids leave in ascending order without a sort.
#include "device.h"

namespace idx {

constexpr int kTopkThreads = 256;
constexpr int kPerThread = IDX_MAX_BLOCKS / kTopkThreads;  // 32

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;  // NaN
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* wave_tot) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) wave_tot[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = wave_tot[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / 64; ++w) m = min(m, wave_tot[w]);
  __syncthreads();
  return m;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const StepArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kTopkThreads / 64];
  __shared__ uint32_t pick_digit, pick_above, pick_count;

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

  // this thread's blocks and keys
  const int C = (nb + kTopkThreads - 1) / kTopkThreads;
  const int b0 = tid * C;
  const int cnt = max(0, min(C, nb - b0));
  const int init = a.init_blocks, local_from = nb - a.local_blocks;
  float sv[kPerThread];
  uint32_t key[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) sv[j] = (j < cnt) ? bs[b0 + j] : 0.0f;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nforced = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int b = b0 + j;
    const bool forced = b < init || b >= local_from;
    key[j] = order_key(sv[j]);
    if (j < cnt && !forced) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
    nforced += (j < cnt && forced) ? 1u : 0u;
  }
  uint32_t total;
  block_exclusive_scan<kTopkThreads>(nforced, wave_tot, &total);
  const uint32_t F = total;
  kmin = block_min_u32(kmin, wave_tot);
  kmax = ~block_min_u32(~kmax, wave_tot);

  // radix select of the want-th largest non-forced key
  uint32_t want = (uint32_t)K - F;  // the free slots (F <= init + local <= K)
  uint32_t prefix = kmin, tshift = 0;
  if (want > 0 && kmin != kmax) {
    int hi = 31 - __builtin_clz(kmin ^ kmax);
    prefix = (hi == 31) ? 0u : (kmin >> (hi + 1)) << (hi + 1);
    while (hi >= 0) {
      const int lo = max(hi - 7, 0);
      const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int b = b0 + j;
        const bool forced = b < init || b >= local_from;
        const uint32_t k = key[j];
        const bool match = (hi == 31) || ((k >> (hi + 1)) == (prefix >> (hi + 1)));
        if (j < cnt && !forced && match) atomicAdd(&hist[(k >> lo) & dmask], 1u);
      }
      __syncthreads();
      // thread t looks at digit 255 - t: counts of larger digits come first
      const uint32_t h = hist[255 - tid];
      uint32_t tot;
      const uint32_t above = block_exclusive_scan<kTopkThreads>(h, wave_tot, &tot);
      if (above < want && want <= above + h) {
        pick_digit = 255u - (uint32_t)tid;
        pick_above = above;
        pick_count = h;
      }
      __syncthreads();
      prefix |= pick_digit << lo;
      want -= pick_above;
      tshift = (uint32_t)lo;
      const bool done = (pick_count == want);  // the whole bin is taken
      __syncthreads();
      if (done) break;
      hi = lo - 1;
    }
  }
  const uint32_t T = prefix >> tshift;

  // positions: forced and > T are taken; of the keys == T, the `want` lowest ids
  uint32_t sure = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int b = b0 + j;
    const bool forced = b < init || b >= local_from;
    const uint32_t kt = key[j] >> tshift;
    if (j < cnt) {
      sure += (forced || (want > 0 && kt > T)) ? 1u : 0u;
      eq += (!forced && want > 0 && kt == T) ? 1u : 0u;
    }
  }
  const uint32_t ex = block_exclusive_scan<kTopkThreads>((sure << 16) | eq, wave_tot, &total);
  uint32_t eq_rank = ex & 0xFFFFu;
  uint32_t pos = (ex >> 16) + min(eq_rank, want);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int b = b0 + j;
    const bool forced = b < init || b >= local_from;
    const uint32_t kt = key[j] >> tshift;
    if (j < cnt) {
      bool take = forced || (want > 0 && kt > T);
      if (!forced && want > 0 && kt == T) {
        take = eq_rank < want;
        ++eq_rank;
      }
      if (take && pos < (uint32_t)K) {
        ids[pos] = b;
        sc[pos] = sv[j];
      }
      pos += take ? 1u : 0u;
    }
  }
}

hipError_t launch_topk(const StepArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_req * a.P * a.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace idx
