// attn.hip -- sparse attention over the selected blocks, for gfx950 (MI355X).
//
// The step after selection: each query head of KV head h of a draft row
// attends over the tokens of the blocks index head h selected for that row,
// under the row's own length (sglang PR 45451, Accuracy Tests, runs the sparse
// kernel's tests beside the packed scorer; ROCm/ATOM PR 2745, Validation,
// times the fused verify kernel on MI355X).
//
// Work item = (request, KV head).  Its P draft rows x G query heads (P <= 16,
// P G <= 64) form T = ceil(P G / 16) 16-row MFMA tiles, each wave holding
// all T: every 32-token unit of K and V it loads serves all of them.  The
// item walks the union of its P rows'
// selections, each block carrying the mask of the rows that chose it: a block
// chosen by several draft rows is read from HBM once for all of them, as the
// indexer reads each K page once for all rows of a request.  An item's union
// is cut into `splits` contiguous shares, one workgroup of four waves each
// (one workgroup a CU, so one wave a SIMD); wave w takes the share's blocks w,
// w + 4, ... and keeps its own online-softmax state, the four are merged in LDS, and the workgroup writes
// its partial (max, sum, unnormalized output) per row.  A second kernel merges
// the splits of an item; an item that is not split (splits = 1) writes its
// output directly and no merge runs.
//
// Per 32-token unit of a block, per wave:
//   S^T = K Q^T   MFMA 16x16x32 bf16 with K as the A operand: lane (m, gq)
//                 loads its k positions of token pi_c(m)'s row, so lane (n, gq)
//                 ends with row n's scores of tokens 8 gq .. 8 gq + 7 (two
//                 16-token halves c = 0, 1, pi_c(m) = 8 (m / 4) + 4 c + m % 4);
//   O^T += V^T P^T  with P^T as the B operand, which is exactly what each lane
//                 holds (its row's probabilities of those 8 tokens, in bf16),
//                 and V^T as the A operand, read as 8 contiguous tokens of one
//                 dimension from the unit's transposed V: each 32-token
//                 quarter of a page-head is stored [128 dims][32 tokens], so
//                 one load instruction (16 dimensions) covers whole lines.
// So K and V go from HBM straight into operand registers, and the rescale of
// the running output is local to each lane (lane n holds row n's output
// dimensions 16 dt + 4 gq + i).  Loads go through per-page buffer descriptors;
// a page outside the pool gets an empty one (reads nothing) and makes every
// row that sees it NaN.
//
// K and V in bf16 or in fp8 e4m3 (unit scale, the index cache's fp8 format).
// fp8 bytes are widened exactly to bf16 in registers (every e4m3 value is a
// bf16 value) and go through the same bf16 products, so only the bytes read
// change.  Which head dimensions a lane feeds at k-step s (Q read to match;
// the dot product does not depend on the order of its terms):
//   bf16  K row 256 B, four 16-byte loads:  d = 32 s + 8 gq .. + 8
//   fp8   K row 128 B, two 16-byte loads at bytes 16 gq and 64 + 16 gq:
//         d = 64 (s / 2) + 16 gq + 8 (s % 2) .. + 8
// and V's 8 tokens of a dimension are 16 bytes (bf16) or 8 bytes (fp8).
#include <algorithm>
#include <atomic>

#include "device.h"

namespace idx {

// Tuning knobs (compile-time; neither changes what is computed).
#ifndef IDX_ATTN_RING
#define IDX_ATTN_RING 3      // 32-token units in registers per wave, bf16 K/V (64 registers each)
#endif
#ifndef IDX_ATTN_RING_FP8
#define IDX_ATTN_RING_FP8 4  // the same for fp8 K/V (32 registers each)
#endif
#ifndef IDX_ATTN_MIN_WGS
#define IDX_ATTN_MIN_WGS 1   // workgroups a CU must hold at once (sets each wave's register budget)
#endif

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnBitWords = IDX_MAX_BLOCKS / 32;
constexpr int kPartFloats = 132;  // per row of a partial: output [0, 128), max (log2 units), sum, pad
constexpr float kAttnLazy = 8.f;  // log2 units a row's max may pass its reference before a rescale

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// One page-head of K (and of V): 128 tokens x 128 dimensions.
template <int KVF>
constexpr int kPageHeadBytes = KVF == IDX_K_BF16 ? 32768 : 16384;

template <int KVF>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const uint8_t* pool, int64_t page_head, bool ok) {
  const uint8_t* base = ok ? pool + page_head * kPageHeadBytes<KVF> : pool;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, ok ? kPageHeadBytes<KVF> : 0,
                                           0x00020000);
}

// One 32-token unit of a block in a lane's registers.
template <int KVF>
struct AttnUnit;
template <>
struct AttnUnit<IDX_K_BF16> {
  static constexpr int kRing = IDX_ATTN_RING;
  u32x4 k[2][4];  // [half c][k-step s]
  u32x4 v[8];     // [dim tile dt]
};
template <>
struct AttnUnit<IDX_K_FP8_E4M3> {
  static constexpr int kRing = IDX_ATTN_RING_FP8;
  u32x4 k[2][2];  // [half c][16-byte load i]: k-steps 2 i, 2 i + 1
  u32x2 v[8];     // [dim tile dt]
};

// Eight e4m3 bytes (lo: the first four) widened to bf16 (exact, scale 1).
__device__ __forceinline__ bf16x8_t widen_fp8x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The K operand of half c, k-step s, and the V operand of dimension tile dt.
__device__ __forceinline__ bf16x8_t k_operand(const AttnUnit<IDX_K_BF16>& w, int c, int s) {
  return __builtin_bit_cast(bf16x8_t, w.k[c][s]);
}
__device__ __forceinline__ bf16x8_t k_operand(const AttnUnit<IDX_K_FP8_E4M3>& w, int c, int s) {
  const u32x4 x = w.k[c][s >> 1];
  return (s & 1) ? widen_fp8x8(x.z, x.w) : widen_fp8x8(x.x, x.y);
}
__device__ __forceinline__ bf16x8_t v_operand(const AttnUnit<IDX_K_BF16>& w, int dt) {
  return __builtin_bit_cast(bf16x8_t, w.v[dt]);
}
__device__ __forceinline__ bf16x8_t v_operand(const AttnUnit<IDX_K_FP8_E4M3>& w, int dt) {
  return widen_fp8x8(w.v[dt].x, w.v[dt].y);
}

// First head dimension of the 8 that a lane of k-group gq feeds at k-step s.
template <int KVF>
__device__ __forceinline__ int attn_d0(int s, int gq) {
  return KVF == IDX_K_BF16 ? 32 * s + 8 * gq : 64 * (s >> 1) + 16 * gq + 8 * (s & 1);
}

// Row `row` (of the item's P x G) of item (request r, KV head h): output
// dimensions 8 c8 .. + 8 from the unnormalized sum acc8 over all its tokens,
// with running max M (log2 units) and sum L; NaN when a bad page was seen.
__device__ __forceinline__ void attn_finalize(const AttnArgs& a, int r, int h, int row, int c8, float M, float L,
                                              const float* acc8, bool nan) {
  const int j = row / a.G, g = row - j * a.G;
  const int64_t orow = (((int64_t)(r * a.P + j)) * a.H + h) * a.G + g;
  bf16x8_t ob;
  float lse;
  if (nan) {
#pragma unroll
    for (int d = 0; d < 8; ++d) ob[d] = (__bf16)__builtin_nanf("");
    lse = __builtin_nanf("");
  } else if (M == -INFINITY) {
#pragma unroll
    for (int d = 0; d < 8; ++d) ob[d] = (__bf16)0.f;
    lse = -INFINITY;
  } else {
    const float inv = 1.f / L;
#pragma unroll
    for (int d = 0; d < 8; ++d) ob[d] = (__bf16)(acc8[d] * inv);
    lse = (M + __builtin_amdgcn_logf(L)) * 0.693147180559945309f;
  }
  *reinterpret_cast<bf16x8_t*>(a.out + orow * 128 + 8 * c8) = ob;
  if (c8 == 0) a.lse[orow] = lse;
}

// Ring depth for T query tiles a wave: the tiles' outputs and queries take
// the registers a deeper ring would.
template <int KVF, int T>
constexpr int attn_ring() {
  return T == 1 ? AttnUnit<KVF>::kRing : (KVF == IDX_K_BF16 ? 2 : 3);
}

// Whether the running output is rescaled lazily (see compute below), by
// measurement: it pays where the vector work and the registers are tight
// (fp8 widening, several tiles, the tiles' outputs held in AGPRs), and costs
// where they are not or where it pushes the register allocation into spills.
template <int KVF, int T>
constexpr bool attn_lazy() {
  return KVF == IDX_K_FP8_E4M3 ? T >= 2 : T == 3;
}

template <int KVF, int T>
__global__ __launch_bounds__(kAttnThreads, IDX_ATTN_MIN_WGS) void attn_partial_kernel(const AttnArgs a) {
  typedef AttnUnit<KVF> Unit;
  constexpr int kRing = attn_ring<KVF, T>();
  __shared__ int32_t list_id[IDX_ATTN_MAX_IDS];
  __shared__ int32_t list_page[IDX_ATTN_MAX_IDS];
  __shared__ uint16_t list_mask[IDX_ATTN_MAX_IDS];
  __shared__ union {
    uint32_t bits[IDX_ATTN_MAX_DRAFT][kAttnBitWords];  // each draft row's selected blocks
    struct {
      float o[kAttnWaves][16][128];  // one 16-row tile at a time
      float m[kAttnWaves][16];
      float l[kAttnWaves][16];
    } comb;
  } U;
  __shared__ uint32_t wave_tot[kAttnWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)__builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.splits;
  const int item = blockIdx.x / S, split = blockIdx.x - item * S;
  const int H = a.H, P = a.P, G = a.G, MB = a.max_blocks, K = a.topk;
  const int r = item / H, h = item - r * H;
  const int nw = (MB + 31) >> 5;
  const int slot = a.req_slot[r];
  const bool pad = slot < 0 || slot >= a.n_slot_rows;

  // 1. each draft row's selected blocks it can see, as bitmaps
  for (int x = tid; x < P * kAttnBitWords; x += kAttnThreads) U.bits[x / kAttnBitWords][x % kAttnBitWords] = 0u;
  __syncthreads();
  if (!pad) {
    for (int e = tid; e < P * K; e += kAttnThreads) {
      const int j = e / K;
      const int nb = blocks_of(clamp_len(a.row_len[r * P + j], MB));
      const int id = a.topk_ids[((int64_t)(r * P + j) * H + h) * K + (e - j * K)];
      if (id >= 0 && id < nb) atomicOr(&U.bits[j][id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  // 2. their union in ascending id order, each block with its row mask
  uint32_t u = 0;
  if (tid < nw)
    for (int j = 0; j < P; ++j) u |= U.bits[j][tid];
  uint32_t nu;
  uint32_t pos = block_exclusive_scan<kAttnThreads>((uint32_t)__builtin_popcount(u), wave_tot, &nu);
  for (uint32_t x = u; x; x &= x - 1) {
    const int bit = __builtin_ctz(x);
    uint32_t mask = 0;
    for (int j = 0; j < P; ++j) mask |= ((U.bits[j][tid] >> bit) & 1u) << j;
    list_id[pos] = tid * 32 + bit;
    list_mask[pos] = (uint16_t)mask;
    ++pos;
  }
  __syncthreads();
  // 3. this workgroup's share of the union and its page ids
  const int lo = (int)((int64_t)split * nu / S), hi = (int)((int64_t)(split + 1) * nu / S);
  for (int x = lo + tid; x < hi; x += kAttnThreads) list_page[x] = a.block_table[(int64_t)slot * MB + list_id[x]];
  __syncthreads();

  // 4. the wave's blocks: lo + wave, lo + wave + 4, ... A fixed assignment
  // keeps the order of every floating-point sum, so repeated calls give
  // bit-identical outputs; with one wave a SIMD it measured as fast as
  // handing blocks out from an LDS counter.  Tile t holds rows 16 t .. 16 t
  // + 15 of the item's P x G; lane n of it is row 16 t + n.
  const int n = lane & 15, gq = lane >> 4;
  bf16x8_t qf[T][4];
  int my_len[T];
  uint32_t jbit[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int rr = 16 * t + n;
    const bool row_ok = rr < P * G;
    const int j = row_ok ? rr / G : 0, g = row_ok ? rr - j * G : 0;
    const int64_t qrow = (((int64_t)(r * P + j)) * H + h) * G + g;
    my_len[t] = row_ok && !pad ? clamp_len(a.row_len[r * P + j], MB) : 0;
    jbit[t] = row_ok ? (1u << j) : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (row_ok) w = *reinterpret_cast<const u32x4*>(a.q + qrow * 128 + attn_d0<KVF>(s, gq));
      qf[t][s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int my_blocks = (hi - lo - wave + kAttnWaves - 1) / kAttnWaves;  // may be <= 0
  const int n_units = my_blocks > 0 ? 4 * my_blocks : 0;

  float m[T], l[T];
  bool bad[T];
  f32x4 o[T][8];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
    bad[t] = false;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // token of K row this lane loads for half c: pi_c(n)
  const int tk0 = 8 * (n >> 2) + (n & 3);

  auto issue = [&](Unit& w, int U_) {
    const int x = lo + wave + kAttnWaves * (U_ >> 2);
    const bool exists = U_ < n_units;
    const int page = exists ? (int)__builtin_amdgcn_readfirstlane((uint32_t)list_page[x]) : -1;
    const bool ok = exists && page >= 0 && page < a.n_pages;
    const int64_t ph = (int64_t)(ok ? page : 0) * H + h;
    const __amdgpu_buffer_rsrc_t rk = attn_rsrc<KVF>(a.k, ph, ok);
    const __amdgpu_buffer_rsrc_t rv = attn_rsrc<KVF>(a.v, ph, ok);
    const int sub = U_ & 3;
    if constexpr (KVF == IDX_K_BF16) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          w.k[c][s] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (32 * sub + tk0 + 4 * c) * 256 + 64 * s + 16 * gq, 0, 0));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)  // V quarter `sub`: [128 dims][32 tokens], 64 B a dimension
        w.v[dt] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 8192 * sub + (16 * dt + n) * 64 + 16 * gq, 0, 0));
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          w.k[c][i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (32 * sub + tk0 + 4 * c) * 128 + 64 * i + 16 * gq, 0, 0));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)  // V quarter `sub`: [128 dims][32 tokens], 32 B a dimension
        w.v[dt] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, 4096 * sub + (16 * dt + n) * 32 + 8 * gq, 0, 0));
    }
  };

  auto compute = [&](const Unit& w, int U_) {
    if (U_ >= n_units) return;
    const int x = lo + wave + kAttnWaves * (U_ >> 2);
    const int b = (int)__builtin_amdgcn_readfirstlane((uint32_t)list_id[x]);
    const uint32_t mask = __builtin_amdgcn_readfirstlane((uint32_t)list_mask[x]);
    const int page = (int)__builtin_amdgcn_readfirstlane((uint32_t)list_page[x]);
    const bool ok = page >= 0 && page < a.n_pages;
    // the unit's operands, widened once for all tiles
    bf16x8_t ko[2][4], vo[8];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 4; ++s) ko[c][s] = k_operand(w, c, s);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vo[dt] = v_operand(w, dt);
    // this lane: row 16 t + n, tokens 8 gq + 4 c + i of the unit
    const int pos0 = 128 * b + 32 * (U_ & 3) + 8 * gq;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bool sel = (mask & jbit[t]) != 0u;
      bad[t] |= sel && !ok;
      f32x4 acc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ko[c][s], qf[t][s], acc[c], 0, 0, 0);
      }
      float xv[8];
      float mt = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = sel && ok && pos0 + 4 * c + i < my_len[t];
          xv[4 * c + i] = vis ? acc[c][i] * a.c2 : -INFINITY;
          mt = fmaxf(mt, xv[4 * c + i]);
        }
      mt = fmaxf(mt, x16(mt, gq));
      mt = fmaxf(mt, x32(mt, gq));
      // Lazy (attn_lazy): the exponentials are taken against a reference m
      // that moves only when some row's max passes it by more than
      // kAttnLazy (then every row of the tile moves to its true max and its
      // sums are rescaled), so most units leave the running output alone; a
      // weight is then at most 2^kAttnLazy, well inside bf16 and fp32, and
      // the final normalisation uses the same m.  Otherwise m follows the
      // max at every unit.
      if (!attn_lazy<KVF, T>() || __builtin_amdgcn_ballot_w64(mt > m[t] + kAttnLazy) != 0) {
        const float mn = fmaxf(m[t], mt);
        const float alpha = mn != -INFINITY ? __builtin_amdgcn_exp2f(m[t] - mn) : 1.f;
        l[t] *= alpha;
        m[t] = mn;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
      }
      const bool live = m[t] != -INFINITY;  // some token of this row seen so far
      float sum = 0.f;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = live ? __builtin_amdgcn_exp2f(xv[e] - m[t]) : 0.f;
        sum += pe;
        pb[e] = (__bf16)pe;
      }
      l[t] += sum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo[dt], pb, o[t][dt], 0, 0, 0);
    }
  };

  {
    Unit ring[kRing];
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) issue(ring[k], k);
    for (int U0 = 0; U0 < n_units; U0 += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        issue(ring[(k + kRing - 1) % kRing], U0 + k + kRing - 1);
        compute(ring[k], U0 + k);
      }
    }
  }

  // 5. per tile, merge the four waves in LDS (the bitmaps are dead) and
  // write the partial (or, unsplit, the output)
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float lt = l[t];
    lt += x16(lt, gq);
    lt += x32(lt, gq);
    __syncthreads();
    if (gq == 0) {
      U.comb.m[wave][n] = m[t];
      U.comb.l[wave][n] = bad[t] ? __builtin_nanf("") : lt;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&U.comb.o[wave][n][16 * dt + 4 * gq]) = o[t][dt];
    __syncthreads();
    const int row = tid >> 4, c8 = tid & 15;  // row of the tile
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      M = fmaxf(M, U.comb.m[w2][row]);
      nan |= U.comb.l[w2][row] != U.comb.l[w2][row];
    }
    float L = 0.f, acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float mw = U.comb.m[w2][row];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * U.comb.l[w2][row];
#pragma unroll
      for (int d = 0; d < 8; ++d) acc8[d] += f * U.comb.o[w2][row][8 * c8 + d];
    }
    const int irow = 16 * t + row;  // row of the item
    if (S == 1) {  // the whole union: the output itself
      if (irow < P * G) attn_finalize(a, r, h, irow, c8, M, L, acc8, nan);
      continue;
    }
    if (nan) L = __builtin_nanf("");
    float* part = a.ws + (((int64_t)item * S + split) * 16 * T + irow) * kPartFloats;
    if (c8 == 0) {
      part[128] = M;
      part[129] = L;
    }
    *reinterpret_cast<f32x4*>(part + 8 * c8) = f32x4{acc8[0], acc8[1], acc8[2], acc8[3]};
    *reinterpret_cast<f32x4*>(part + 8 * c8 + 4) = f32x4{acc8[4], acc8[5], acc8[6], acc8[7]};
  }
}

// Merge the splits of each item: row 16 t + tid / 16 writes output
// dimensions 8 (tid % 16) .. + 8 (and its lse), t over the item's T tiles.
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(const AttnArgs a, int T) {
  const int item = blockIdx.x, tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, S = a.splits;
  const int r = item / H, h = item - r * H;
  const int c8 = tid & 15;
  const int64_t step = (int64_t)16 * T * kPartFloats;  // one split further
  for (int t = 0; t < T; ++t) {
    const int row = 16 * t + (tid >> 4);
    if (row >= P * G) break;  // rows grow with t
    const float* part = a.ws + ((int64_t)item * S * 16 * T + row) * kPartFloats;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const float* ps = part + s * step;
      M = fmaxf(M, ps[128]);
      nan |= ps[129] != ps[129];
    }
    float L = 0.f, acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll 8
      for (int s = 0; s < S; ++s) {
        const float* ps = part + s * step;
        const float f = (ps[128] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ps[128] - M);
        L += f * ps[129];
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(ps + 8 * c8);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(ps + 8 * c8 + 4);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc8[d] += f * v0[d];
          acc8[4 + d] += f * v1[d];
        }
      }
    }
    attn_finalize(a, r, h, row, c8, M, L, acc8, nan);
  }
}

namespace {
// Every instantiation has the same register and LDS budget (one workgroup a
// CU); the bf16 one-tile one is asked.
int attn_resident_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int nwg = cache[dev].load(std::memory_order_relaxed); nwg > 0) return nwg;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(attn_partial_kernel<IDX_K_BF16, 1>),
                                                   kAttnThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev].store(cus * per_cu, std::memory_order_relaxed);
  return cus * per_cu;
}
}  // namespace

int attn_splits(int64_t items, int64_t max_union) {
  if (items <= 0) return 1;
  // enough workgroups to fill the device, but at least 8 blocks a split of
  // the largest union an item can have (a split of nothing still costs its
  // set-up, and the merge one partial more)
  int64_t s = (attn_resident_workgroups() + items - 1) / items;
  s = std::min<int64_t>(s, std::max<int64_t>(1, (max_union + 7) / 8));
  return (int)(s < 1 ? 1 : (s > IDX_ATTN_MAX_SPLITS ? IDX_ATTN_MAX_SPLITS : s));
}

namespace {
template <int KVF, int T>
void launch_partial(const AttnArgs& a, int64_t items, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial_kernel<KVF, T>), dim3((unsigned)(items * a.splits)), dim3(kAttnThreads), 0, stream,
                     a);
}
template <int KVF>
void launch_partial_tiles(const AttnArgs& a, int64_t items, int T, hipStream_t stream) {
  switch (T) {
    case 1: launch_partial<KVF, 1>(a, items, stream); break;
    case 2: launch_partial<KVF, 2>(a, items, stream); break;
    case 3: launch_partial<KVF, 3>(a, items, stream); break;
    default: launch_partial<KVF, 4>(a, items, stream); break;
  }
}
}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.n_req * a.H;
  if (items == 0) return hipSuccess;
  const int T = attn_tiles(a.P, a.G);
  if (a.kv_format == IDX_K_FP8_E4M3)
    launch_partial_tiles<IDX_K_FP8_E4M3>(a, items, T, stream);
  else
    launch_partial_tiles<IDX_K_BF16>(a, items, T, stream);
  if (a.splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)items), dim3(kAttnThreads), 0, stream, a, T);
  return hipGetLastError();
}

}  // namespace idx
