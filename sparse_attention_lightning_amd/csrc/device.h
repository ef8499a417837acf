// device.h -- internal types and helpers of the gfx950 indexer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "idx.h"

namespace idx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kBlock = 128;   // tokens per block = tokens per page
constexpr int kTileRows = 16; // rows of the packed query tile

// Everything the kernels need, by value (one parameter block per launch).
struct StepArgs {
  const void* q;
  const void* k;
  const uint8_t* k_scale;
  const int32_t* req_slot;
  const int32_t* block_table;
  const int32_t* row_len;
  float* block_scores;
  int32_t* topk_ids;
  float* topk_scores;
  int64_t n_pages;
  int32_t k_format;
  int32_t n_req, n_slot_rows, P, H, max_blocks, topk, init_blocks, local_blocks;
  int32_t score_mode;  // IDX_SCORE_MAX or IDX_SCORE_LSE
  float sm_scale;      // lse only
  // NVFP4 only: new keys the score kernel quantizes into the pool (k, k_scale)
  // before it reads them (st_n = 0: none); see the fused store in score.hip
  const uint16_t* st_staging;  // bf16 [st_n][st_stride]
  const int64_t* st_slots;     // [st_n]
  int64_t st_n, st_stride;
};

// Sparse attention over the selected blocks (one launch of partials, one of
// the merge).
struct AttnArgs {
  const uint16_t* q;          // bf16 [R*P][H][G][128]
  const uint8_t* k;           // bf16 or fp8 [n_pages][H][128 tokens][128]
  const uint8_t* v;           // bf16 or fp8 [n_pages][H][4][128 dims][32 tokens]
  const int32_t* req_slot;
  const int32_t* block_table;
  const int32_t* row_len;
  const int32_t* topk_ids;    // [R*P][H][topk]
  uint16_t* out;              // bf16 [R*P][H][G][128]
  float* lse;                 // [R*P][H][G]
  float* ws;                  // partials: [R*H][splits][16 rows][132]
  int64_t n_pages;
  int32_t n_req, n_slot_rows, P, H, G, max_blocks, topk, splits;
  int32_t kv_format;          // IDX_K_BF16 or IDX_K_FP8_E4M3 (K and V alike)
  float c2;                   // sm_scale * log2(e)
};
// Workgroups of the partial kernel per (request, KV head) item, for `items`
// items whose unions hold at most `max_union` blocks.
int attn_splits(int64_t items, int64_t max_union);
// 16-row query tiles of an item's P x G rows.
inline int attn_tiles(int P, int G) { return (P * G + 15) / 16; }
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

hipError_t launch_score(const StepArgs& a, hipStream_t stream);       // any rows per request
hipError_t launch_score_rows(const StepArgs& a, hipStream_t stream);  // more than 16 rows per request
hipError_t launch_topk(const StepArgs& a, hipStream_t stream);
hipError_t launch_fp4_store(const uint16_t* staging, int64_t n_tokens, int64_t stride,
                            const int64_t* slot_mapping, uint8_t* payload, uint8_t* scales,
                            int64_t n_slots, hipStream_t stream);
hipError_t launch_read_probe(const void* base, int64_t n_base_units, const int32_t* units, int64_t n_units,
                             int unit_bytes, bool nt, uint32_t* sink, int n_sink, hipStream_t stream);
// The device address of this device's block-score array of idx_step_noalloc
// (looked up on the first call per device).
hipError_t noalloc_scores(float** out);

__device__ __forceinline__ int clamp_len(int32_t len, int max_blocks) {
  const int cap = max_blocks * kBlock;
  return len < 0 ? 0 : (len > cap ? cap : len);
}

__device__ __forceinline__ int blocks_of(int len) { return (len + kBlock - 1) / kBlock; }

// A value every lane of the wave holds, as a scalar.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Lane permutation within DPP rows (16 lanes); CTRL is the DPP control word.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15), in every lane.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_mov<0x128>(x));  // row_ror:8
  return x;
}

// Sum over the 16 lanes of a DPP row, in every lane (the rotations reach
// offsets 0, 4, 8 and 12 after the quad steps).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x124>(x);  // row_ror:4
  x += dpp_mov<0x128>(x);  // row_ror:8
  return x;
}

// The value lane l ^ 16 (x16) or l ^ 32 (x32) holds, for a lane of lane group
// g = l / 16, through the gfx950 lane swaps (VALU, no LDS round trip): a swap
// of v with itself leaves the partner row's copy in the second result on
// lanes 0-15 and 32-47 (x16) or 0-31 (x32), and in the first on the others.
__device__ __forceinline__ float x16(float v, int g) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((g & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float x32(float v, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((g & 2) ? r[0] : r[1]);
}

// Exclusive prefix sum over a workgroup of THREADS threads (all must call);
// *total receives the full sum.  wave_tot: THREADS / 64 words of LDS.
template <int THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // inclusive sum over the wave with DPP: row_shr within rows of 16 lanes,
  // then row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3
  // (a shifted-out or masked-off lane adds 0)
  uint32_t incl = v;
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) {
    const uint32_t t = wave_tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

}  // namespace idx
