// score_rows.hip -- block scoring of requests with more than 16 rows for
// gfx950 (MI355X): many query rows per request, as the prefill scorer has
// (ATOM PR 2745, Summary: a prefill block scorer beside the decode one), and
// packs wider than one tile (sglang PR 45451, Modifications: the one-tile
// packed form applies while packed_queries x gqa <= 16).
//
// What is computed is the same as for the packed tile: row i of request r is
// (query row i / gqa, head i % gqa) and scores each 128-token block under its
// own length; only the work split differs.  A request's rows are cut into
// groups of 512 (eight waves of 64 rows, four 16-row tiles each) and its
// blocks into chunks; an item is one (request, row group, block chunk).
//
// A workgroup widens each K page of its item to bf16 once, as it copies the
// page into LDS (fp8 e4m3 widens exactly; an NVFP4 value, e2m1 code times its
// E4M3 group scale, has at most five fraction bits and is exact in bf16 too),
// so every format is scored by the same bf16 MFMAs against the request's bf16
// queries, and the eight waves share one decode.  Per 16-token tile and
// 32-element k-step, one MFMA 16x16x32 takes the K tile as its A operand and
// a 16-row query tile as B, so lane l = 16 g + n holds tokens 4g .. 4g+3 of
// query row n: most of the max (or log-sum-exp) over a block is taken inside
// the lane, and one exchange across the four lane groups leaves lane group g
// with the block scores of tile g.  The four tiles of a wave share each K
// operand read from LDS.
//
// Pages reach LDS through a ring of register buffers that keeps the next
// RING - 1 pages' loads in flight while the waves score the current one; past
// the item's last page the ring loads through empty descriptors, so the loop
// has no branches around its loads.  The next page's copy into the second LDS
// buffer runs among the current page's MFMAs.  An item reads K only up to its
// longest row (with causal row lengths, a prefill row at position p sees
// p + 1 tokens, items above the diagonal exit at once) and the C chunks of a
// row group split that extent evenly, so the chunks of a row group are equal
// however long its rows are.  Each XCD takes a contiguous run of items, so
// the workgroups that read the same K pages share an L2.
//
// Max mode: block scores leave in granules of 16 blocks of a row (64 bytes,
// aligned in the array when max_blocks is a multiple of 16).  Each lane puts
// its row's score of a page in LDS (two granule buffers, by granule parity,
// rows consecutive so that a page's scores are one conflict-free write),
// and when an item has scored all its blocks of a granule the workgroup
// writes that granule for all its rows, four lanes a row, 16 rows an
// instruction.  The chunk that ends a row group's extent pads its last
// granule with -inf and writes the -inf past it.  Where whole granules can
// be dealt out to the chunks without lengthening the longest one, chunk
// boundaries fall between granules; otherwise on 16-byte pieces, and a
// granule cut by a boundary is written in two parts by two workgroups (odd
// chunks walk their blocks backwards, so both parts are written at about
// the same time).  The stores are nontemporal: a 128-byte line holds two
// granules, written 16 pages apart, and as ordinary stores its first half
// often left L2 before the second came, so 1.3 times the block-score bytes
// reached HBM on the prefill workload; nontemporal, 1.09 times, in the same
// time.  Values stored one by one as each page was scored, before the
// staging, reached HBM about ten times over (3.3 times with four values a
// 16-byte store).  lse mode stores each score as it is made: it is bound
// by its vector work, the writes do not bound it, and staging cost it 5 %
// (more wait states in its tighter register budget).
#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

#include "tile.h"

namespace idx {

#ifndef IDX_ROWS_RING_BF16
#define IDX_ROWS_RING_BF16 2  // pages in the register ring, bf16 K (16 VGPRs a page)
#endif
#ifndef IDX_ROWS_RING_FP8
#define IDX_ROWS_RING_FP8 4   // fp8 K (8 VGPRs a page)
#endif
#ifndef IDX_ROWS_RING_FP4
#define IDX_ROWS_RING_FP4 4   // NVFP4 K (5 VGPRs a page, with scales)
#endif
#ifndef IDX_ROWS_STORE_AT
#define IDX_ROWS_STORE_AT 3   // max: the next page is copied to LDS after this 16-token tile (0..7);
                              // lse: after the page (its half-page accumulators leave no registers)
#endif

#ifndef IDX_ROWS_ITEMS
#define IDX_ROWS_ITEMS 1      // items per resident workgroup the block chunks aim at
#endif
#ifndef IDX_ROWS_NT_STORE
#define IDX_ROWS_NT_STORE 1   // max: block scores leave with nontemporal stores
#endif
#ifndef IDX_ROWS_GRAN_SPLIT
#define IDX_ROWS_GRAN_SPLIT 1  // max: chunk boundaries between output granules where that costs no time
#endif
// Eight waves of four tiles: two waves a SIMD share the matrix core (one
// wave of eight tiles a SIMD measured a third slower: it cannot keep the
// core busy through its own waits).
constexpr int kRowWaves = 8;
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kWaveTiles = 4;                          // lane group g ends with tiles g, g + 4, ...
constexpr int kWaveRows = kTileRows * kWaveTiles;
constexpr int kItemRows = kWaveRows * kRowWaves;
static_assert(kWaveTiles % 4 == 0, "tiles a wave: a multiple of the four lane groups");
constexpr int kMaxItemBlocks = 1024;                   // blocks of an item at most (page ids in LDS)
constexpr int kPageUnits = kHeadDim * 2 / 16;          // 16-byte units of a bf16 token row (16)
constexpr int kGran = 16;                              // blocks of a row in one 64-byte output granule

// LDS slot of 16-byte unit `unit` of token `tok` in a page: rows of 256 bytes,
// the unit index XORed with the token's low four bits.  Sixteen lanes that
// read one unit of sixteen consecutive tokens (the MFMA operand reads), or
// the units of one row (the page copy), then touch sixteen different bank
// groups; padding the rows by 16 bytes instead measured about four conflict
// cycles per 16-byte read on gfx950.
__device__ __forceinline__ int page_slot(int tok, int unit) { return tok * kPageUnits + (unit ^ (tok & 15)); }

template <int FMT>
constexpr int rows_ring() {
  return FMT == IDX_K_BF16 ? IDX_ROWS_RING_BF16 : FMT == IDX_K_FP8_E4M3 ? IDX_ROWS_RING_FP8 : IDX_ROWS_RING_FP4;
}

// LDS of a workgroup: two bf16 K pages in 16-byte units (typed so that each
// access is one 16-byte LDS instruction), the item's page ids, and each row's
// scores of its current output granule.
struct RowsLds {
  u32x4 page[2][kBlock * kPageUnits];
  int32_t pid[kMaxItemBlocks];
  int32_t nbw[kRowWaves];
  float gran[2][kGran][kItemRows];  // [granule parity][slot][row]: a page's scores are one conflict-free write
};

// A page's bytes in flight in registers: 16-byte pieces, consecutive threads
// on consecutive pieces (bf16: 4 a thread, fp8: 2, NVFP4: 1 plus the two scale
// bytes of its 32 values).
template <int FMT>
struct PageRegs {
  static constexpr int kPieces = kBlock * Fmt<FMT>::kRowBytes / 16 / kRowThreads;
  u32x4 v[kPieces];
  uint32_t s;
};

template <int FMT>
__device__ __forceinline__ void page_load(PageRegs<FMT>& pr, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rs, int tid) {
#pragma unroll
  for (int m = 0; m < PageRegs<FMT>::kPieces; ++m)
    pr.v[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * (tid + kRowThreads * m), 0, 0));
  if constexpr (FMT == IDX_K_NVFP4)  // piece tid = token tid / 4, scale groups 2 (tid % 4), +1
    pr.s = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * tid, 0, 0);
}

// Two fp8 bytes (byte pair HI of w) widened to a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// The two e2m1 codes of byte SEL of w times the group scale, as a bf16 pair.
// The products are exact in f32 and in bf16, so keeping the upper halves of
// the f32 words is the exact conversion.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float scale) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return __builtin_amdgcn_perm(__float_as_uint(v.y * scale), __float_as_uint(v.x * scale), 0x07060302u);
}

// Widen the page in flight to bf16 and write it to LDS page P.
template <int FMT>
__device__ __forceinline__ void page_store(const PageRegs<FMT>& pr, u32x4* P, int tid) {
  if constexpr (FMT == IDX_K_BF16) {
#pragma unroll
    for (int m = 0; m < PageRegs<FMT>::kPieces; ++m) {
      const int piece = tid + kRowThreads * m;  // token piece / 16, unit piece % 16
      P[page_slot(piece >> 4, piece & 15)] = pr.v[m];
    }
  } else if constexpr (FMT == IDX_K_FP8_E4M3) {
#pragma unroll
    for (int m = 0; m < PageRegs<FMT>::kPieces; ++m) {
      const int piece = tid + kRowThreads * m;  // token piece / 8, dims 16 (piece % 8) ..
      const u32x4 w = pr.v[m];
      const int tok = piece >> 3, u0 = 2 * (piece & 7);
      P[page_slot(tok, u0)] = u32x4{fp8_pair<false>(w.x), fp8_pair<true>(w.x), fp8_pair<false>(w.y), fp8_pair<true>(w.y)};
      P[page_slot(tok, u0 + 1)] =
          u32x4{fp8_pair<false>(w.z), fp8_pair<true>(w.z), fp8_pair<false>(w.w), fp8_pair<true>(w.w)};
    }
  } else {
    static_assert(kBlock * Fmt<IDX_K_NVFP4>::kRowBytes == 16 * kRowThreads, "one 16-byte NVFP4 piece a thread");
    // token tid / 4, dims 32 (tid % 4) ..: bytes 0-7 in scale group 2 (tid % 4), bytes 8-15 in the next
    const float s0 = __builtin_amdgcn_cvt_scalef32_f32_fp8(pr.s, 1.0f, 0);
    const float s1 = __builtin_amdgcn_cvt_scalef32_f32_fp8(pr.s, 1.0f, 1);
    const u32x4 w = pr.v[0];
    const int tok = tid >> 2, u0 = 4 * (tid & 3);
    P[page_slot(tok, u0)] = u32x4{fp4_pair<0>(w.x, s0), fp4_pair<1>(w.x, s0), fp4_pair<2>(w.x, s0), fp4_pair<3>(w.x, s0)};
    P[page_slot(tok, u0 + 1)] =
        u32x4{fp4_pair<0>(w.y, s0), fp4_pair<1>(w.y, s0), fp4_pair<2>(w.y, s0), fp4_pair<3>(w.y, s0)};
    P[page_slot(tok, u0 + 2)] =
        u32x4{fp4_pair<0>(w.z, s1), fp4_pair<1>(w.z, s1), fp4_pair<2>(w.z, s1), fp4_pair<3>(w.z, s1)};
    P[page_slot(tok, u0 + 3)] =
        u32x4{fp4_pair<0>(w.w, s1), fp4_pair<1>(w.w, s1), fp4_pair<2>(w.w, s1), fp4_pair<3>(w.w, s1)};
  }
}

// max(a, b) as the median of (a, b, +inf): a NaN operand is dropped as fmaxf
// drops it, and MFMA results need no canonicalizing first (an fmaxf on them
// costs one extra VALU op per value).  The +inf comes from a scalar move the
// compiler cannot see through; with a literal it turns the median back into
// fmaxf.
__device__ __forceinline__ float opaque_inf() {
  float x;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(x));
  return x;
}
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, opaque_inf()); }

// The running block state of this lane's tokens, per tile: IDX_SCORE_MAX
// keeps the max of q.k in m; IDX_SCORE_LSE the max m of v = c2 q.k and
// s = sum of 2^(v - m).
struct BlockState {
  float m[kWaveTiles];
  float s[kWaveTiles];
};

// Two partial log-sum-exp states (max m, sum s of 2^(v - m)) merged.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float base = (mn == -INFINITY) ? 0.f : mn;
  s = s * __builtin_amdgcn_exp2f(m - base) + s2 * __builtin_amdgcn_exp2f(m2 - base);
  m = mn;
}

// lse terms v[0..N) (masked ones -inf) of tile u's row folded into the
// block state against the lane's base ref[u], taking the terms' own max as
// the new base when their sum against the old one leaves [2^-64, 2^64) (0
// included: nothing visible, or no base yet).  The exact path for
// fold_half's exceptions.
template <int N>
__device__ __forceinline__ void fold_terms(const float* v, int u, BlockState& st, float c2, float* ref) {
  float base = ref[u], sum = 0.f;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {  // a second pass only after a new base
    sum = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) sum += __builtin_amdgcn_exp2f(fmaf(v[i], c2, -base));
    // on its own max the sum lies in [1, N], unless a dot is NaN or
    // infinite: then the NaN it gives is kept
    if (((sum >= 0x1p-64f) & (sum < 0x1p64f)) | (pass == 1)) break;
    float am = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i) am = max2(am, v[i]);
    base = am * c2;  // -inf * c2 = -inf
    if (base == -INFINITY) {  // nothing visible
      sum = 0.f;
      break;
    }
  }
  if (sum != 0.f) {
    ref[u] = base;
    if (st.m[u] == base) {
      st.s[u] += sum;
    } else if (st.m[u] == -INFINITY) {
      st.m[u] = base;
      st.s[u] = sum;
    } else {
      lse_merge(st.m[u], st.s[u], base, sum);
    }
  }
}

// Fold one half page's dot products (acc[u][t][e]: tile u's row n against
// token 16 t + 4 g + e of the half, whose block position is pos0 + 16 t + e)
// into the state.  len[u]: the length of tile u's row n.  FULL: every token
// of the block is visible to every row of the wave (no masks).
// lse: each lane keeps a base ref[u] for tile u's row from block to block;
// the half's terms 2^(c2 v - ref) are summed against it and, while the
// sums stay in [2^-64, 2^64) and the block's state is on the same base,
// simply added (no max, no rescaling).  Otherwise the exact path makes the
// terms' own max the base.  c2 m + log2 s does not depend on the base, and
// inside that window no term that matters underflows and none overflows.
template <int MODE, bool FULL>
__device__ __forceinline__ void fold_half(const f32x4 (*acc)[4], int pos0, const int* len, BlockState& st,
                                          float c2, float* ref) {
  float v[kWaveTiles][16];
#pragma unroll
  for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[u][4 * t + e] = (FULL || pos0 + 16 * t + e < len[u]) ? acc[u][t][e] : -INFINITY;
  if constexpr (MODE == IDX_SCORE_MAX) {
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u) {
      float am = v[u][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) am = max2(am, v[u][i]);
      st.m[u] = fmaxf(st.m[u], am);
    }
  } else {
    float sum[kWaveTiles];
    bool fast = true;
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u) {
      const float nb = -ref[u];
      sum[u] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum[u] += __builtin_amdgcn_exp2f(fmaf(v[u][i], c2, nb));
      fast = fast & (sum[u] >= 0x1p-64f) & (sum[u] < 0x1p64f) & ((st.m[u] == ref[u]) | (st.m[u] == -INFINITY));
    }
    if (__builtin_amdgcn_ballot_w64(!fast) == 0) {  // every lane: its sums on its bases, as they are
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u) {
        st.s[u] = ((st.m[u] == -INFINITY) ? 0.f : st.s[u]) + sum[u];
        st.m[u] = ref[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u) fold_terms<16>(v[u], u, st, c2, ref);
    }
  }
}

// Reduce the values of tiles Q .. Q+3 over the four lane groups (lanes n,
// n + 16, n + 32, n + 48) so that lane group g ends with tile Q + g's: two
// exchange steps, each lane keeping half of what it holds and receiving the
// partner's copy of it.
template <int MODE, int Q>
__device__ __forceinline__ void group_reduce(const BlockState& st, int g, float& m, float& s) {
  const bool o1 = g & 1, o2 = g & 2;
  float a_m[2], a_s[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // keep tiles Q + (g & 1) and Q + 2 + (g & 1), send the others
    a_m[i] = o1 ? st.m[Q + 2 * i + 1] : st.m[Q + 2 * i];
    const float rm = x16(o1 ? st.m[Q + 2 * i] : st.m[Q + 2 * i + 1], g);
    if constexpr (MODE == IDX_SCORE_MAX) {
      a_m[i] = fmaxf(a_m[i], rm);
    } else {
      a_s[i] = o1 ? st.s[Q + 2 * i + 1] : st.s[Q + 2 * i];
      const float rs = x16(o1 ? st.s[Q + 2 * i] : st.s[Q + 2 * i + 1], g);
      lse_merge(a_m[i], a_s[i], rm, rs);
    }
  }
  // a[0]: tile g & 1, a[1]: tile 2 + (g & 1), over groups g, g ^ 1
  m = o2 ? a_m[1] : a_m[0];
  const float rm = x32(o2 ? a_m[0] : a_m[1], g);
  if constexpr (MODE == IDX_SCORE_MAX) {
    m = fmaxf(m, rm);
    s = 0.f;
  } else {
    s = o2 ? a_s[1] : a_s[0];
    const float rs = x32(o2 ? a_s[0] : a_s[1], g);
    lse_merge(m, s, rm, rs);
  }
}

// One item (all threads of the workgroup; every early return is taken by the
// whole workgroup).  G row groups a request, C block chunks a row group.
template <int FMT, int MODE>
__device__ __forceinline__ void score_item(const StepArgs& a, RowsLds& L, int item, int G, int C) {
  constexpr int kPageBytes = kBlock * Fmt<FMT>::kRowBytes;
  constexpr int D = rows_ring<FMT>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uniform((uint32_t)(tid >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int gi = item % G, rc = item / G, c = rc % C, r = rc / C;
  const int PH = a.P * a.H, MB = a.max_blocks;
  const int slot = a.req_slot[r];
  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  const int wrow0 = gi * kItemRows + kWaveRows * wave;  // the wave's first row in the request

  // lengths: row n of each tile, and row 16 g + n (the row this lane scores
  // out); rows past the request have none
  auto row_len = [&](int i) -> int {
    const int row = wrow0 + i;
    return (row < PH && !pad) ? clamp_len(a.row_len[r * a.P + row / a.H], MB) : 0;
  };
  int len[kWaveTiles];
  int nbw = 0, lmin = INT_MAX;
#pragma unroll
  for (int u = 0; u < kWaveTiles; ++u) {
    len[u] = row_len(kTileRows * u + n);
    nbw = max(nbw, blocks_of(len[u]));
    if (wrow0 + kTileRows * u + n < PH) lmin = min(lmin, len[u]);
  }
  int my_len[kWaveTiles / 4];  // row 16 (4 q + g) + n, scored out by this lane
#pragma unroll
  for (int q = 0; q < kWaveTiles / 4; ++q) my_len[q] = row_len(kTileRows * (4 * q + g) + n);
  // the wave's extent and its shortest real row (full blocks skip the masks)
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    nbw = max(nbw, __shfl_xor(nbw, o));
    lmin = min(lmin, __shfl_xor(lmin, o));
  }
  nbw = (int)uniform((uint32_t)nbw);
  lmin = (int)uniform((uint32_t)lmin);
  if (lane == 0) L.nbw[wave] = nbw;
  __syncthreads();
  int nb_item = 0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) nb_item = max(nb_item, L.nbw[w]);
  nb_item = (int)uniform((uint32_t)nb_item);

  // The end (exclusive) of the output granule holding a row's last scored
  // block, capped at the row's end: the chunk that scores that block fills
  // the granule's rest with -inf.  Blocks from there on (past the row
  // group's longest row, every block of a graph pad) get -inf from the
  // chunk-0 workgroup of the row group.
  constexpr bool kStaged = MODE == IDX_SCORE_MAX;  // lse stores each score as it is made (see the header)
  // chunk c of C: an even share of the row group's own extent, so the items
  // of a row group do the same work whatever its rows' lengths; in max mode
  // the inner boundaries are rounded to multiples of four blocks, so the
  // parts of a granule two chunks write are whole 16-byte pieces (at most
  // kMaxItemBlocks blocks: the launch makes ceil(max_blocks / C) + 4 no more)
  // When whole granules can be dealt out to the C chunks without making the
  // row group's largest chunk longer than ceil(max_blocks / C) (the chunk
  // the launch sized for), the boundaries fall between granules and no
  // granule is written in two parts.
  const int ngran = (nb_item + kGran - 1) / kGran;
  const bool gran_split = IDX_ROWS_GRAN_SPLIT && kStaged &&
                          kGran * ((ngran + C - 1) / C) <= (MB + C - 1) / C;
  auto chunk_start = [&](int cc) -> int {
    if (cc >= C) return nb_item;
    if (gran_split) return min(nb_item, kGran * (int)((int64_t)cc * ngran / C));
    const int x = (int)((int64_t)cc * nb_item / C);
    return kStaged ? min(nb_item, (x + 2) & ~3) : x;
  };
  const int b0 = chunk_start(c);
  const int nblk = chunk_start(c + 1) - b0;
  // blocks past the row group's longest row (every block of a graph pad) get
  // -inf from the chunk that ends the extent (chunk 0 when there is none);
  // with aligned granules its last one is padded, and the rest starts whole
  const bool whole = kStaged && (MB % kGran) == 0 && (reinterpret_cast<uintptr_t>(a.block_scores) & 15) == 0;
  const bool ends = (nb_item == 0) ? (c == 0) : (nblk > 0 && b0 + nblk == nb_item);
  // max mode: block scores leave with nontemporal stores (see the header)
  constexpr bool kNt = kStaged && IDX_ROWS_NT_STORE;
  if (ends) {
    const int fill_from = whole ? min(MB, (nb_item + kGran - 1) & ~(kGran - 1)) : nb_item;
    for (int i = 0; i < kWaveRows; ++i) {
      const int row = wrow0 + i;
      if (row >= PH) break;
      float* out = a.block_scores + ((int64_t)r * PH + row) * MB;
      for (int b = fill_from + lane; b < MB; b += 64) {
        if constexpr (kNt)
          __builtin_nontemporal_store(-INFINITY, out + b);
        else
          out[b] = -INFINITY;
      }
    }
  }
  if (nblk <= 0) return;
  const bool rev = kStaged && (c & 1) != 0;  // odd chunks take their blocks last to first
  auto blk = [&](int k) -> int { return b0 + (rev ? nblk - 1 - k : k); };  // the block of the k-th page
  const bool active = wrow0 < PH;  // the wave has rows
  for (int j = tid; j < nblk; j += kRowThreads) L.pid[j] = a.block_table[(int64_t)slot * MB + b0 + j];

  // the wave's query tiles as B operands: row n of tile u, k-step s = dims
  // d0(s, g) .. +8, the one-tile kernel's order for the format (the K operand
  // reads the same dims), so both kernels sum the same products in the same
  // order
  bf16x8 qf[kWaveTiles][4];
#pragma unroll
  for (int u = 0; u < kWaveTiles; ++u) {
    const int row = wrow0 + kTileRows * u + n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < PH)
        v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                            ((int64_t)r * PH + row) * kHeadDim + Fmt<FMT>::d0(s, g));
      qf[u][s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float c2 = (MODE == IDX_SCORE_LSE) ? a.sm_scale * 1.44269504088896341f : 0.f;
  float ref[kWaveTiles];  // lse: each tile row's base for its terms (+inf: none yet)
#pragma unroll
  for (int u = 0; u < kWaveTiles; ++u) ref[u] = INFINITY;
  // the item's blocks gl .. gh of granule G (blocks 16 G .. 16 G + 15; at
  // the extent's end padded with -inf to the granule's end), written by the
  // whole workgroup: four lanes a row, 16 rows an instruction
  auto write_granule = [&](int G, int gl, int gh) {
    const int ge = (ends && whole && gh == nb_item - 1) ? kGran * G + kGran - 1 : gh;
    float* base = a.block_scores + ((int64_t)r * PH + gi * kItemRows) * MB + kGran * G;
#pragma unroll 1
    for (int x = tid; x < kItemRows * (kGran / 4); x += kRowThreads) {
      const int lr = x >> 2, e = x & 3;
      if (gi * kItemRows + lr >= PH) break;  // x grows with the row
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = L.gran[G & 1][4 * e + i][lr];
      float* dst = base + (int64_t)lr * MB + 4 * e;
      const int b1 = kGran * G + 4 * e;  // the block of v[0]
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (b1 + i <= gh) ? v[i] : -INFINITY;
      if (whole) {  // the item's blocks of a granule are whole 16-byte pieces
        if (b1 >= gl && b1 <= ge) {
          if constexpr (kNt)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          else
            *reinterpret_cast<f32x4*>(dst) = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (b1 + i >= gl && b1 + i <= ge) dst[i] = v[i];
      }
    }
  };
  // after the pages k0 .. k1 - 1: the granules whose blocks of this item are
  // now all scored (at most two)
  auto write_done = [&](int k0, int k1) {
    const int lo = rev ? b0 + nblk - k1 : b0, hi = rev ? b0 + nblk - 1 : b0 + k1 - 1;  // scored so far
    const int pl = rev ? lo : b0 + k0, ph = rev ? b0 + nblk - 1 - k0 : hi;             // by these pages
    for (int G = pl / kGran; G <= ph / kGran; ++G) {
      const int gl = max(kGran * G, b0), gh = min(kGran * G + kGran - 1, b0 + nblk - 1);
      if (gl >= lo && gh <= hi) write_granule(G, gl, gh);
    }
  };

  // page j of the item: its id (-1 past the item) and descriptors
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  auto page_of = [&](int k) -> int { return (k < nblk) ? L.pid[rev ? nblk - 1 - k : k] : -1; };
  auto issue = [&](PageRegs<FMT>& pr, int pid) {
    const bool ok = pid >= 0 && pid < a.n_pages;
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(kp, pid, ok, kPageBytes);
    const __amdgpu_buffer_rsrc_t rs = (FMT == IDX_K_NVFP4) ? page_rsrc(a.k_scale, pid, ok, kBlock * 8) : rk;
    page_load<FMT>(pr, rk, rs, tid);
  };

  // tile T's K operands (16 tokens x the four k-steps) from LDS page P
  auto k_ops = [&](const u32x4* P, int T, u32x4* ko) {
#pragma unroll
    for (int s = 0; s < 4; ++s) ko[s] = P[page_slot(16 * T + n, Fmt<FMT>::d0(s, g) / 8)];
  };
  // the page's eight 16-token tiles against the wave's four query tiles
  // (acc[u]: tile u's row n x tokens 16 T + 4 g .. +3), the next tile's K
  // operands read while this one's MFMAs run; max folds each tile as it is
  // done, lse a half page at a time (against each row's base: no max, no
  // rescaling)
  auto page_dots = [&](const u32x4* P, auto full_tag, int b, BlockState& st, auto&& mid) {
    constexpr bool FULL = decltype(full_tag)::value;
    u32x4 ko[2][4];
    f32x4 acch[kWaveTiles][4];
    k_ops(P, 0, ko[0]);
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      if (T + 1 < 8) k_ops(P, T + 1, ko[(T + 1) & 1]);
      f32x4 acc[kWaveTiles];
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < kWaveTiles; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ko[T & 1][s]), qf[u][s],
                                                           acc[u], 0, 0, 0);
      const int pos0 = b * kBlock + 16 * T + 4 * g;  // block position of acc[u][0]
      if constexpr (MODE == IDX_SCORE_MAX) {
#pragma unroll
        for (int u = 0; u < kWaveTiles; ++u) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (FULL || pos0 + e < len[u]) ? acc[u][e] : -INFINITY;
          st.m[u] = max2(st.m[u], max2(max2(v[0], v[1]), max2(v[2], v[3])));
        }
      } else {
#pragma unroll
        for (int u = 0; u < kWaveTiles; ++u) acch[u][T & 3] = acc[u];
        if ((T & 3) == 3) fold_half<MODE, FULL>(acch, pos0 - 48, len, st, c2, ref);
      }
      if constexpr (MODE == IDX_SCORE_MAX)
        if (T == IDX_ROWS_STORE_AT) mid();
    }
  };
  // mid(): the next page's copy into the other LDS buffer, placed among this
  // page's MFMAs so that its conversions and LDS writes overlap them
  auto score_page = [&](int k, int pid, auto&& mid) {
    const int b = blk(k);
    const u32x4* P = L.page[k & 1];
    BlockState st;
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u) {
      st.m[u] = -INFINITY;
      st.s[u] = 0.f;
    }
    // a wave-uniform branch: blocks every row of the wave sees whole skip
    // the per-token masks
    if ((b + 1) * kBlock <= lmin)
      page_dots(P, std::true_type{}, b, st, mid);
    else
      page_dots(P, std::false_type{}, b, st, mid);
    const bool ok = pid >= 0 && pid < a.n_pages;
    auto out = [&](auto q_tag) {
      constexpr int q = decltype(q_tag)::value;
      float m, s;
      group_reduce<MODE, 4 * q>(st, g, m, s);
      float o;
      if constexpr (MODE == IDX_SCORE_MAX)
        o = m;
      else
        o = (m == -INFINITY) ? -INFINITY : (m + __builtin_amdgcn_logf(s)) * 0.693147180559945309f;
      if (!ok) o = (b * kBlock < my_len[q]) ? __builtin_nanf("") : -INFINITY;
      if constexpr (kStaged) {
        L.gran[(b / kGran) & 1][b & (kGran - 1)][kWaveRows * wave + kTileRows * (4 * q + g) + n] = o;
      } else {
        const int row = wrow0 + kTileRows * (4 * q + g) + n;
        if (row < PH) a.block_scores[((int64_t)r * PH + row) * MB + b] = o;
      }
    };
    out(std::integral_constant<int, 0>{});
    if constexpr (kWaveTiles > 4) out(std::integral_constant<int, 1>{});
    static_assert(kWaveTiles <= 8, "tiles a wave: at most 8");
    if constexpr (MODE == IDX_SCORE_LSE) mid();
  };

  // the ring: slot u holds page k (k % D == u) from its issue D - 1 steps
  // ahead until it is widened into LDS page k & 1
  __syncthreads();  // page ids
  PageRegs<FMT> ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], page_of(u));
  page_store<FMT>(ring[0], L.page[0], tid);
  __syncthreads();
  static_assert(D <= kGran, "a ring pass finishes at most two granules");
  for (int k0 = 0; k0 < nblk; k0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int k = k0 + u;
      const int pid = page_of(k);
      if (u == 0 || k < nblk) {  // (u == 0: k < nblk by the loop bound)
        issue(ring[u], page_of(k + D));  // slot u's page k is in LDS already
        auto store_next = [&] { page_store<FMT>(ring[(u + 1) % D], L.page[(k + 1) & 1], tid); };
        if (active)
          score_page(k, pid, store_next);
        else
          store_next();
      }
      __syncthreads();
    }
    // granules finished by this pass go out (the next pass writes the other
    // granule buffer; this one is reused only 16 blocks later)
    if constexpr (kStaged) write_done(k0, min(k0 + D, nblk));
  }
}

// A resident grid walks the M = n_req * C * G items; the workgroups of each
// XCD (w, w + 8, ... when the grid is a multiple of 8) take a contiguous run.
template <int FMT, int MODE>
__global__ __launch_bounds__(kRowThreads) void rows_kernel(const StepArgs a, int G, int C, int M) {
  __shared__ RowsLds L;
  const int per = (M + 7) / 8;
  for (int x = blockIdx.x; x < 8 * per; x += gridDim.x) {
    const int item = (x % 8) * per + x / 8;
    if (item < M) score_item<FMT, MODE>(a, L, item, G, C);
    __syncthreads();  // LDS free for the next item
  }
}

namespace {
// Workgroups that fit on the device at once (cached per device).
template <int FMT, int MODE>
int rows_resident() {
  static std::atomic<int> cache[64];  // zero-initialised; calls from several threads store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int n = cache[dev].load(std::memory_order_relaxed); n > 0) return n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(rows_kernel<FMT, MODE>),
                                                   kRowThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev].store(cus * per_cu, std::memory_order_relaxed);
  return cus * per_cu;
}

template <int FMT, int MODE>
void launch_rows(const StepArgs& a, hipStream_t stream) {
  const int PH = a.P * a.H;
  const int G = (PH + kItemRows - 1) / kItemRows;
  // block chunks: about IDX_ROWS_ITEMS items per resident workgroup (an item
  // loads its query tiles and page ids and fills its ring once, so items
  // should not be short), at most kMaxItemBlocks blocks each
  const int slots = rows_resident<FMT, MODE>();
  const int64_t groups = (int64_t)a.n_req * G;
  const int64_t want = std::max<int64_t>(1, (IDX_ROWS_ITEMS * (int64_t)slots + groups - 1) / groups);
  const int CB = (int)std::min<int64_t>(kMaxItemBlocks - 4, std::max<int64_t>(1, (a.max_blocks + want - 1) / want));
  const int C = (a.max_blocks + CB - 1) / CB;
  const int64_t M = groups * C;
  const int64_t grid = std::min<int64_t>(8 * ((M + 7) / 8), 8 * ((slots + 7) / 8));
  hipLaunchKernelGGL((rows_kernel<FMT, MODE>), dim3((unsigned)grid), dim3(kRowThreads), 0, stream, a, G, C, (int)M);
}

template <int MODE>
void launch_rows_mode(const StepArgs& a, hipStream_t stream) {
  switch (a.k_format) {
    case IDX_K_BF16: launch_rows<IDX_K_BF16, MODE>(a, stream); break;
    case IDX_K_FP8_E4M3: launch_rows<IDX_K_FP8_E4M3, MODE>(a, stream); break;
    default: launch_rows<IDX_K_NVFP4, MODE>(a, stream); break;
  }
}
}  // namespace

hipError_t launch_score_rows(const StepArgs& a, hipStream_t stream) {
  if (a.n_req == 0 || a.max_blocks == 0) return hipSuccess;
  if (a.score_mode == IDX_SCORE_LSE)
    launch_rows_mode<IDX_SCORE_LSE>(a, stream);
  else
    launch_rows_mode<IDX_SCORE_MAX>(a, stream);
  return hipGetLastError();
}

}  // namespace idx
