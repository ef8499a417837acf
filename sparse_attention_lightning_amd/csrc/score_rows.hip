// score_rows.hip -- block scoring of requests with more than 16 rows for
// gfx950 (MI355X): many query rows per request, as the prefill scorer has
// (ATOM PR 2745, Summary: a prefill block scorer beside the decode one), and
// packs wider than one tile (sglang PR 45451, Modifications: the one-tile
// packed form applies while packed_queries x gqa <= 16).
//
// What is computed is the same as for the packed tile: row i of request r is
// (query row i / gqa, head i % gqa) and scores each 128-token block under its
// own length; only the work split differs.  A request's rows are cut into
// groups of 256 (eight waves, each two 16-row tiles that share every decoded K
// operand) and its blocks into chunks; an item is one (request, row group,
// block chunk).  A workgroup stages each K page of its item in LDS once, and
// the four waves score their tiles against it with the tile code of the
// packed kernel, so a page crosses L2 once per 256 rows and the matrix cores,
// not the memory, bound the kernel.  Pages reach LDS through a ring of
// register buffers that keeps the next RING - 1 pages' loads in flight while
// the waves score the current one; past the item's last page the ring loads
// through empty descriptors, so the loop has no branches around its loads.
// An item reads K only up to its longest row: with causal row lengths (a
// prefill row at position p sees p + 1 tokens) items above the diagonal exit
// at once.  Items are numbered request, then block chunk, then row group, and
// each XCD takes a contiguous run of them, so the workgroups that read the
// same K pages share an L2.  Each wave stages its rows' scores in LDS and
// writes them out every 32 blocks as one 128-byte run per row.
#include <algorithm>
#include <climits>

#include "tile.h"

namespace idx {

#ifndef IDX_ROWS_RING_BF16
#define IDX_ROWS_RING_BF16 3  // pages in the register ring, bf16 K (16 VGPRs a page)
#endif
#ifndef IDX_ROWS_RING_FP8
#define IDX_ROWS_RING_FP8 6   // fp8 K (8 VGPRs a page)
#endif
#ifndef IDX_ROWS_RING_FP4
#define IDX_ROWS_RING_FP4 6   // NVFP4 K (8 VGPRs a page, with scales)
#endif
constexpr int kRowWaves = 8;
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kWaveTiles = 2;                               // 16-row tiles a wave
constexpr int kItemRows = kTileRows * kWaveTiles * kRowWaves;  // 256
constexpr int kStageBlocks = 32;                            // blocks staged between write-outs
constexpr int kMaxItemBlocks = 1024;                        // blocks of an item at most (page ids in LDS)

template <int FMT>
constexpr int rows_ring() {
  return FMT == IDX_K_BF16 ? IDX_ROWS_RING_BF16 : FMT == IDX_K_FP8_E4M3 ? IDX_ROWS_RING_FP8 : IDX_ROWS_RING_FP4;
}

// One K page in LDS, in 16-byte units (typed so that every access is one
// 16-byte LDS instruction): token rows padded by 16 bytes so that the 16
// lanes of a k-group, which read 16 different tokens at one column, fall in
// different banks.
template <int FMT>
struct PageLds {
  static constexpr int kStride = Fmt<FMT>::kRowBytes / 16 + 1;  // 16-byte units per token row
  u32x4 k[kBlock * kStride];
  u32x4 sc[FMT == IDX_K_NVFP4 ? kBlock * 8 / 16 : 1];
};

template <int FMT>
struct RowsLds {
  PageLds<FMT> page[2];
  float stage[kRowWaves][kWaveTiles * kTileRows][kStageBlocks];
  int32_t pid[kMaxItemBlocks];  // the item's page ids
  int32_t nbw[kRowWaves];
};

// A page's bytes in flight in registers: 16-byte pieces, consecutive threads
// on consecutive pieces.
template <int FMT>
struct PageRegs {
  static constexpr int kPieces = kBlock * Fmt<FMT>::kRowBytes / 16 / kRowThreads;
  u32x4 v[kPieces];
  u32x4 s;  // NVFP4: 16 bytes of the page's scale plane (threads < 64)
};

template <int FMT>
__device__ __forceinline__ void page_load(PageRegs<FMT>& pr, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rs, int tid) {
#pragma unroll
  for (int m = 0; m < PageRegs<FMT>::kPieces; ++m)
    pr.v[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * (tid + kRowThreads * m), 0, 0));
  if constexpr (FMT == IDX_K_NVFP4)  // threads >= 64 read past the 1 KB plane: zeros, no memory touched
    pr.s = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * tid, 0, 0));
}

template <int FMT>
__device__ __forceinline__ void page_store(const PageRegs<FMT>& pr, PageLds<FMT>& P, int tid) {
  constexpr int kPerRow = Fmt<FMT>::kRowBytes / 16;  // pieces per token row
#pragma unroll
  for (int m = 0; m < PageRegs<FMT>::kPieces; ++m) {
    const int piece = tid + kRowThreads * m;
    P.k[(piece / kPerRow) * PageLds<FMT>::kStride + piece % kPerRow] = pr.v[m];
  }
  if constexpr (FMT == IDX_K_NVFP4)
    if (tid < kBlock * 8 / 16) P.sc[tid] = pr.s;
}

// One lane's share of half page `half` from LDS, in the layout load_half
// gives from HBM.
template <int FMT>
__device__ __forceinline__ void half_from_lds(Half<FMT>& h, const PageLds<FMT>& P, int half, int n, int g) {
  const int tok0 = half * 64 + n;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = (tok0 + 16 * t) * PageLds<FMT>::kStride;
#pragma unroll
    for (int i = 0; i < Fmt<FMT>::kLoads; ++i) h.v[t][i] = P.k[row + Fmt<FMT>::off(i, g) / 16];
    if constexpr (FMT == IDX_K_NVFP4)
      h.sc[t] = reinterpret_cast<const uint16_t*>(P.sc)[(tok0 + 16 * t) * 4 + g];
  }
}

// One item (all threads of the workgroup; every early return is taken by the
// whole workgroup).  G row groups a request, C chunks of CB blocks each.
template <int FMT, int MODE>
__device__ __forceinline__ void score_item(const StepArgs& a, RowsLds<FMT>& L, int item, int G, int C, int CB) {
  typedef typename Fmt<FMT>::Op Op;
  constexpr int kPageBytes = kBlock * Fmt<FMT>::kRowBytes;
  constexpr int D = rows_ring<FMT>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uniform((uint32_t)(tid >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int gi = item % G, rc = item / G, c = rc % C, r = rc / C;
  const int PH = a.P * a.H, MB = a.max_blocks;
  const int slot = a.req_slot[r];
  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  const int wrow0 = gi * kItemRows + kWaveTiles * kTileRows * wave;  // the wave's first row in the request

  // lengths of tile u: this lane's rows 4g + e, and row 4g + n for a writer
  // lane (n < 4); rows past the request have none
  auto row_len = [&](int i) -> int {
    const int row = wrow0 + i;
    return (row < PH && !pad) ? clamp_len(a.row_len[r * a.P + row / a.H], MB) : 0;
  };
  int len[kWaveTiles][4], my_len[kWaveTiles];
  int nbw = 0, lmin = INT_MAX;
#pragma unroll
  for (int u = 0; u < kWaveTiles; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) len[u][e] = row_len(kTileRows * u + 4 * g + e);
    my_len[u] = (n == 0) ? len[u][0] : (n == 1) ? len[u][1] : (n == 2) ? len[u][2] : len[u][3];
    const int ln = row_len(kTileRows * u + n);
    nbw = max(nbw, blocks_of(ln));
    if (wrow0 + kTileRows * u + n < PH) lmin = min(lmin, ln);
  }
  // the wave's extent and its shortest real row (the fast path skips masks)
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

  // blocks no item covers (past the row group's longest row, every block of a
  // graph pad) get -inf from the chunk-0 workgroup of the row group
  if (c == 0) {
    for (int i = 0; i < kWaveTiles * kTileRows; ++i) {
      const int row = wrow0 + i;
      if (row >= PH) break;
      float* out = a.block_scores + ((int64_t)r * PH + row) * MB;
      for (int b = nb_item + lane; b < MB; b += 64) out[b] = -INFINITY;
    }
  }
  const int b0 = c * CB;
  if (b0 >= nb_item) return;
  const int nblk = min(CB, nb_item - b0);
  const bool active = wrow0 < PH;  // the wave has rows
  for (int j = tid; j < nblk; j += kRowThreads) L.pid[j] = a.block_table[(int64_t)slot * MB + b0 + j];

  // the wave's query tiles (bf16, or f16 under 2^sigma for NVFP4; one sigma
  // for both tiles)
  Op qf[kWaveTiles][4];
  int sigma = 0;
  float c2 = 0.f;  // lse: sm_scale * log2 e * 2^-sigma
  {
    u32x4 pc[kWaveTiles][4];
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pc[u][s] = u32x4{0u, 0u, 0u, 0u};
        const int row = wrow0 + kTileRows * u + n;
        if (row < PH)
          pc[u][s] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                     ((int64_t)r * PH + row) * kHeadDim + Fmt<FMT>::d0(s, g));
      }
    if constexpr (FMT == IDX_K_NVFP4) {
      float m = 0.f;
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            m = fmaxf(m, fmaxf(fabsf(__uint_as_float(pc[u][s][w] << 16)),
                               fabsf(__uint_as_float(pc[u][s][w] & 0xFFFF0000u))));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (m > 0.f) {
        int ex;
        frexpf(m, &ex);  // m < 2^ex
        sigma = 15 - ex;
      }
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const _Float16 lo16 = (_Float16)ldexpf(__uint_as_float(pc[u][s][w] << 16), sigma);
            const _Float16 hi16 = (_Float16)ldexpf(__uint_as_float(pc[u][s][w] & 0xFFFF0000u), sigma);
            pc[u][s][w] = (uint32_t)__builtin_bit_cast(uint16_t, lo16) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, hi16) << 16);
          }
    }
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[u][s] = __builtin_bit_cast(Op, pc[u][s]);
  }
  if constexpr (MODE == IDX_SCORE_LSE) c2 = ldexpf(a.sm_scale * 1.44269504088896341f, -sigma);

  // page j of the item: its id (-1 past the item) and descriptors
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  auto page_of = [&](int j) -> int { return (j < nblk) ? L.pid[j] : -1; };
  auto issue = [&](PageRegs<FMT>& pr, int pid) {
    const bool ok = pid >= 0 && pid < a.n_pages;
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(kp, pid, ok, kPageBytes);
    const __amdgpu_buffer_rsrc_t rs = (FMT == IDX_K_NVFP4) ? page_rsrc(a.k_scale, pid, ok, kBlock * 8) : rk;
    page_load<FMT>(pr, rk, rs, tid);
  };

  const int wrow = 4 * g + n;  // lanes n < 4 hold row 4g + n of each tile
  auto score_page = [&](int k, int pid) {
    const int b = b0 + k;
    const PageLds<FMT>& P = L.page[k & 1];
    float st0[kWaveTiles][4], st1[kWaveTiles][4];
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st0[u][e] = -INFINITY;
        st1[u][e] = 0.f;
      }
    const bool full = (b + 1) * kBlock <= lmin;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      Half<FMT> h;
      half_from_lds<FMT>(h, P, half, n, g);
      f32x4 acc[kWaveTiles][4];
      half_dot<FMT, kWaveTiles>(h, qf, acc);
#pragma unroll
      for (int u = 0; u < kWaveTiles; ++u)
        fold<MODE>(acc[u], full, b * kBlock + 64 * half + n, len[u], st0[u], st1[u], c2);
    }
    const bool ok = pid >= 0 && pid < a.n_pages;
#pragma unroll
    for (int u = 0; u < kWaveTiles; ++u) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float m = row16_max(st0[u][e]);
        if constexpr (MODE == IDX_SCORE_MAX) {
          v[e] = m;
        } else {
          const float base = (m == -INFINITY) ? 0.f : m;
          const float sum = row16_sum(st1[u][e] * __builtin_amdgcn_exp2f(st0[u][e] - base));
          v[e] = (m == -INFINITY) ? -INFINITY : (m + __builtin_amdgcn_logf(sum)) * 0.693147180559945309f;
        }
      }
      float o = (n == 0) ? v[0] : (n == 1) ? v[1] : (n == 2) ? v[2] : v[3];
      if constexpr (FMT == IDX_K_NVFP4 && MODE == IDX_SCORE_MAX) o = ldexpf(o, -sigma);
      if (!ok) o = (b * kBlock < my_len[u]) ? __builtin_nanf("") : -INFINITY;
      if (n < 4) L.stage[wave][kTileRows * u + wrow][k % kStageBlocks] = o;
    }
    // every 32 blocks, and after the last: the wave's rows out as runs
    if (k % kStageBlocks == kStageBlocks - 1 || k == nblk - 1) {
      const int k0 = k - k % kStageBlocks, cnt = k - k0 + 1;
      for (int i = 0; i < kWaveTiles * kTileRows; ++i) {
        const int row = wrow0 + i;
        if (row >= PH) break;
        if (lane < cnt) a.block_scores[((int64_t)r * PH + row) * MB + b0 + k0 + lane] = L.stage[wave][i][lane];
      }
    }
  };

  // the ring: slot u holds page k (k % D == u) from its issue D - 1 steps
  // ahead until it is copied to LDS buffer k & 1
  __syncthreads();  // page ids
  PageRegs<FMT> ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], page_of(u));
  page_store<FMT>(ring[0], L.page[0], tid);
  __syncthreads();
  for (int k0 = 0; k0 < nblk; k0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int k = k0 + u;
      const int pid = page_of(k);
      if (u == 0 || k < nblk) {  // (u == 0: k < nblk by the loop bound)
        issue(ring[u], page_of(k + D));  // slot u's page k is in LDS already
        if (active) score_page(k, pid);
        page_store<FMT>(ring[(u + 1) % D], L.page[(k + 1) & 1], tid);
      }
      __syncthreads();
    }
  }
}

// A resident grid walks the M = n_req * C * G items; the workgroups of each
// XCD (w, w + 8, ... when the grid is a multiple of 8) take a contiguous run.
template <int FMT, int MODE>
__global__ __launch_bounds__(kRowThreads) void rows_kernel(const StepArgs a, int G, int C, int CB, int M) {
  __shared__ RowsLds<FMT> L;
  const int per = (M + 7) / 8;
  for (int x = blockIdx.x; x < 8 * per; x += gridDim.x) {
    const int item = (x % 8) * per + x / 8;
    if (item < M) score_item<FMT, MODE>(a, L, item, G, C, CB);
    __syncthreads();  // LDS free for the next item
  }
}

namespace {
// Workgroups that fit on the device at once (cached per device).
template <int FMT, int MODE>
int rows_resident() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(rows_kernel<FMT, MODE>),
                                                   kRowThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev] = cus * per_cu;
  return cache[dev];
}

template <int FMT, int MODE>
void launch_rows(const StepArgs& a, hipStream_t stream) {
  const int PH = a.P * a.H;
  const int G = (PH + kItemRows - 1) / kItemRows;
  // block chunks: about two items per resident workgroup (an item loads its
  // query tiles and page ids once, so items should not be short), at most
  // kMaxItemBlocks blocks each
  const int slots = rows_resident<FMT, MODE>();
  const int64_t groups = (int64_t)a.n_req * G;
  const int64_t want = std::max<int64_t>(1, (2 * (int64_t)slots + groups - 1) / groups);
  const int CB = (int)std::min<int64_t>(kMaxItemBlocks, std::max<int64_t>(1, (a.max_blocks + want - 1) / want));
  const int C = (a.max_blocks + CB - 1) / CB;
  const int64_t M = groups * C;
  const int64_t grid = std::min<int64_t>(8 * ((M + 7) / 8), 8 * ((slots + 7) / 8));
  hipLaunchKernelGGL((rows_kernel<FMT, MODE>), dim3((unsigned)grid), dim3(kRowThreads), 0, stream, a, G, C, CB,
                     (int)M);
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
