// fp4_store.hip -- NVFP4 index-key store for gfx950.
//
// ROCm/ATOM PR 2745, Summary ("Store" and the per-key layout): per 16-element
// group, scale = e4m3(amax / 6) and codes rounded half-to-even, saturating at
// 6; two codes a byte, the even element in the low nibble; 64 B payload and
// 8 B scales per key, written at the key's slot.
//
// Eight threads per key, one per 16-element group (from 65,536 keys on, four
// threads a key, two groups each); the quantizer itself is in fp4_quant.h,
// shared with the score kernel's fused store of a step's new keys.
#include "fp4_quant.h"

namespace idx {

#ifndef IDX_STORE_UNROLL
#define IDX_STORE_UNROLL 1  // 16-element groups a thread loads before it quantizes them
#endif
#ifndef IDX_STORE_WIDE_MIN
#define IDX_STORE_WIDE_MIN 65536  // keys from which four lanes a key store them (fewer, wider accesses)
#endif
#ifndef IDX_STORE_WIDE_LANES
#define IDX_STORE_WIDE_LANES 4  // lanes a key of the large-store kernel (4 or 2)
#endif
#ifndef IDX_STORE_GRID_CAP
#define IDX_STORE_GRID_CAP 32768  // most workgroups a store launches (threads then stride over the keys)
#endif
#ifndef IDX_STORE_WIDE_UNROLL
#define IDX_STORE_WIDE_UNROLL 2  // large-store kernel: keys a thread loads before it quantizes any
#endif
#ifndef IDX_STORE_NT
#define IDX_STORE_NT 0      // 1: non-temporal staging loads and payload / scale stores
#endif

constexpr int kStoreThreads = 256;

// KL lanes a key, 8 / KL groups a lane: lane q of the key loads its 256 / KL
// bytes of staging and stores its 64 / KL bytes of payload as 16-byte
// pieces; lane 0 of the key stores the 8 scale bytes.  For large stores:
// fewer, wider accesses a key.  The whole 150K NVFP4 pool (9.87 M keys)
// stored in 692 us with four lanes a key, 727 with eight (the other kernel)
// and 769 with two (medians of 36 interleaved calls, one box); a thread
// loading two keys before it quantizes either, on at most 32,768
// workgroups, then took it from 687 to 667 us (one key a thread on 65,536:
// the former; 16,384 or 8,192 workgroups, or three keys a thread, were no
// better).  A small store (a step's 256 new keys) keeps eight lanes a key:
// with one group a lane its chain is shortest, and a small grid has no
// bandwidth to win.
template <int KL>
__global__ __launch_bounds__(kStoreThreads) void fp4_store_wide_kernel(
    const uint16_t* __restrict__ staging, int64_t n_tokens, int64_t stride,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ payload,
    uint8_t* __restrict__ scales, int64_t n_slots) {
  constexpr int NG = 8 / KL;  // groups a lane
  constexpr int U = IDX_STORE_WIDE_UNROLL;
  const int64_t n_items = n_tokens * KL;
  const int64_t step = (int64_t)gridDim.x * kStoreThreads;
  for (int64_t item0 = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x; item0 < n_items; item0 += step * U) {
    u32x4 w[U][2 * NG];
    int64_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = item0 + u * step;
      slot[u] = -1;
      if (item < n_items) {  // a key's KL items are all in range or all out (n_items is a multiple of KL)
        const int64_t t = item / KL;
        const int q = (int)(item % KL);
        const u32x4* src = reinterpret_cast<const u32x4*>(staging + t * stride + 16 * NG * q);
#pragma unroll
        for (int i = 0; i < 2 * NG; ++i) w[u][i] = src[i];
        slot[u] = slot_mapping[t];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = item0 + u * step;
      if (item >= n_items || slot[u] < 0 || slot[u] >= n_slots) continue;  // the key's lanes skip it together
      const int q = (int)(item % KL);
      uint32_t p[2 * NG], sw = 0;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) sw |= quantize16(w[u][2 * gi], w[u][2 * gi + 1], &p[2 * gi]) << (8 * (gi & 3));
#pragma unroll
      for (int i = 0; i < NG / 2; ++i)
        *reinterpret_cast<u32x4*>(payload + slot[u] * 64 + 16 * (NG / 2) * q + 16 * i) =
            u32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
      uint32_t lo, hi;
      if constexpr (KL == 4) {  // lanes 0, 1 of the quad make bytes 0..3, lanes 2, 3 bytes 4..7
        uint32_t word = sw << (16 * (q & 1));
        word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        lo = word;
        hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
      } else {  // lane 0 bytes 0..3, lane 1 bytes 4..7
        lo = sw;
        hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sw, 0xB1, 0xF, 0xF, false);
      }
      if (q == 0) *reinterpret_cast<u32x2*>(scales + slot[u] * 8) = u32x2{lo, hi};
    }
  }
}

// Eight lanes a key, one per group; a thread takes IDX_STORE_UNROLL items a
// grid-stride step and issues all their loads before quantizing any.
__global__ __launch_bounds__(kStoreThreads) void fp4_store_kernel(
    const uint16_t* __restrict__ staging, int64_t n_tokens, int64_t stride,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ payload,
    uint8_t* __restrict__ scales, int64_t n_slots) {
  constexpr int U = IDX_STORE_UNROLL;
  const int64_t n_items = n_tokens * 8;
  const int64_t step = (int64_t)gridDim.x * kStoreThreads;
  for (int64_t item0 = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x; item0 < n_items; item0 += step * U) {
    u32x4 w0[U], w1[U];
    int64_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = item0 + u * step;
      slot[u] = -1;
      if (item < n_items) {  // a key's 8 items are all in range or all out (n_items is a multiple of 8)
        const int64_t t = item >> 3;
        const int grp = (int)(item & 7);
        // the key's row is read whether or not its slot is valid, so the
        // loads overlap (the row is in range either way)
        const u32x4* src = reinterpret_cast<const u32x4*>(staging + t * stride + 16 * grp);
        if constexpr (IDX_STORE_NT) {
          w0[u] = __builtin_nontemporal_load(src);
          w1[u] = __builtin_nontemporal_load(src + 1);
        } else {
          w0[u] = src[0];
          w1[u] = src[1];
        }
        slot[u] = slot_mapping[t];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = item0 + u * step;
      if (item < n_items && slot[u] >= 0 && slot[u] < n_slots)  // the key's 8 lanes take this together
        quantize_group<IDX_STORE_NT != 0>(w0[u], w1[u], slot[u], (int)(item & 7), payload, scales);
    }
  }
}

hipError_t launch_fp4_store(const uint16_t* staging, int64_t n_tokens, int64_t stride,
                            const int64_t* slot_mapping, uint8_t* payload, uint8_t* scales,
                            int64_t n_slots, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if (n_tokens >= IDX_STORE_WIDE_MIN) {
    constexpr int KL = IDX_STORE_WIDE_LANES;
    const int64_t want = (n_tokens * KL + (int64_t)kStoreThreads * IDX_STORE_WIDE_UNROLL - 1) /
                         ((int64_t)kStoreThreads * IDX_STORE_WIDE_UNROLL);
    const unsigned grid = (unsigned)(want < IDX_STORE_GRID_CAP ? want : IDX_STORE_GRID_CAP);
    hipLaunchKernelGGL(fp4_store_wide_kernel<KL>, dim3(grid), dim3(kStoreThreads), 0, stream, staging,
                       n_tokens, stride, slot_mapping, payload, scales, n_slots);
    return hipGetLastError();
  }
  const int64_t want = (n_tokens * 8 + (int64_t)kStoreThreads * IDX_STORE_UNROLL - 1) /
                       ((int64_t)kStoreThreads * IDX_STORE_UNROLL);
  const unsigned grid = (unsigned)(want < IDX_STORE_GRID_CAP ? want : IDX_STORE_GRID_CAP);
  hipLaunchKernelGGL(fp4_store_kernel, dim3(grid), dim3(kStoreThreads), 0, stream, staging,
                     n_tokens, stride, slot_mapping, payload, scales, n_slots);
  return hipGetLastError();
}

}  // namespace idx
