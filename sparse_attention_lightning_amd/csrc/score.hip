// score.hip -- packed block scoring for gfx950 (MI355X).
//
// All of a request's rows (packed_queries x gqa <= 16) form one 16-row MFMA
// tile, so each K page is read from HBM once for every row and head (sglang
// PR 45451, Modifications; sglang PR 42614, Modifications item 1).  The K read
// extent is the group's longest row; masks use each row's own length.  A
// request whose slot lies outside the request table is a graph pad: it reads
// no K.
//
// Work split.  One workgroup of eight waves per CU stays resident for the
// whole launch.  The pages of the step, in (request, block) order, are cut
// into contiguous shares, one per workgroup: equal ones, or, for shares of
// 4 MiB of K and more once every workgroup has reported, sized by the rate each XCD reached on
// the previous launch (XCDs stream at rates a few per cent apart, so equal
// shares leave the slower ones finishing last).  A workgroup takes its
// share in rounds of at most 768 pages touching at most 8 requests.  A round
// first stages its page ids, the query tiles and row lengths of its requests
// in LDS; the eight waves then take pages one at a time from an LDS counter,
// so a wave that is served faster by the memory system simply takes more
// pages (the two waves of a SIMD do not get equal shares of its memory
// pipeline: the older one runs about twice as fast).  Pages are handed out in
// order of their place in the pool (a counting sort of the round's page ids
// into 256 equal buckets of the pool): every workgroup's share is spread over
// the whole pool, so all workgroups then sweep it from its low pages to its
// high ones together, which the memory system serves faster than the same
// pages in random order.  Each page's 16 row scores go to an LDS stage, and
// after a barrier the whole workgroup writes the round's block scores out as
// runs of consecutive blocks per row, so the output leaves in whole 128-byte
// lines.
//
// The 16-row tile, the lane mapping and the per-format k assignment are in
// tile.h.  Each wave streams its pages as 64-token halves through a ring of
// register buffers, keeping RING - 1 halves in flight while the matrix cores
// work on one.
#include <atomic>
#include <climits>
#include <cstddef>

#include "fp4_quant.h"
#include "tile.h"

namespace idx {

#ifndef IDX_SCORE_SORT_BUCKETS
#define IDX_SCORE_SORT_BUCKETS 256  // page-id buckets of the pool for the hand-out order (0: round order)
#endif
#ifndef IDX_SCORE_SORT_MIN
#define IDX_SCORE_SORT_MIN 32       // rounds with fewer pages keep round order
#endif
#ifndef IDX_SCORE_ADAPT
#define IDX_SCORE_ADAPT 1        // shares follow the XCDs' measured page rates (see below)
#endif
#ifndef IDX_SCORE_ADAPT_MIN_BYTES
#define IDX_SCORE_ADAPT_MIN_BYTES (4 << 20)  // K bytes a workgroup from which they do (below, fixed
#endif                                       // costs and vector work blur the XCDs' memory rates)
#ifndef IDX_SCORE_NT_OUT
#define IDX_SCORE_NT_OUT 0       // 1: non-temporal block-score stores
#endif
#ifndef IDX_SCORE_WAVES
#define IDX_SCORE_WAVES 8        // waves of a workgroup (one workgroup a CU)
#endif
constexpr int kWaves = IDX_SCORE_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kPagesPerThread = (768 + kThreads - 1) / kThreads;  // round pages a thread stages
constexpr int kQPiecesPerThread = (8 * 16 * 16) / kThreads;       // query-tile pieces a thread loads
constexpr int kRoundPages = 768;   // pages a workgroup stages at once
constexpr int kRoundReqs = 8;      // requests a round may touch
constexpr int kQStride = 136;      // 16-bit values per query row in LDS (272 B: rows change banks)
constexpr uint32_t kSkNewKeys = 0x2000u;  // sk bit: the page holds new NVFP4 keys (fused store)
constexpr int kKeysPerThread = (IDX_FP4_FUSED_MAX_KEYS + kThreads - 1) / kThreads;  // fused store: slots a thread holds

// ---------------------------------------------------------------------------
// Rounds.  A workgroup's range of the step's pages is handled in rounds of at
// most kRoundPages pages touching at most kRoundReqs requests (one round at
// the sizes served); a round's page ids, query tiles, row lengths and block
// scores live in LDS.

struct RoundReq {
  int32_t r, p0, nbg, lmin;  // request, its first page in step order, its pages, shortest row
  int32_t sigma, pad0, pad1, pad2;
  int32_t len[kTileRows];    // each row's clamped length, 0 past the request's rows
};

struct RoundLds {
  float stage[kTileRows][kRoundPages];            // block scores of the round
  int32_t pid[kRoundPages];                       // page ids, in hand-out order
  uint16_t sk[kRoundPages];                       // in hand-out order: round page | request in the round << 10
                                                  // | kSkNewKeys
  uint8_t ridx[kRoundPages];                      // each round page's request within the round
  uint16_t q[kRoundReqs][kTileRows][kQStride];    // query tiles (bf16, or f16 scaled by 2^sigma)
  RoundReq req[kRoundReqs];
  uint32_t amax[kRoundReqs];                      // NVFP4: largest |q| of each tile (float bits)
  uint32_t next;                                  // pages handed out
  uint32_t wave_tot[kWaves];                      // scan scratch
  // NVFP4 with new keys (the fused store): the keys whose page this round
  // reads (their pages carry kSkNewKeys in sk), and whether wave 0 has
  // stored them
  uint16_t own[IDX_FP4_FUSED_MAX_KEYS];
  uint32_t n_own, keys_ready;
};
static_assert(offsetof(RoundLds, q) % 16 == 0 && offsetof(RoundLds, req) % 16 == 0, "16-byte LDS rows");
// with the per-request arrays for the largest request count, one workgroup
// still fits in the 160 KB of LDS of a CU
static_assert(sizeof(RoundLds) + 64 + (2 * IDX_MAX_REQ + 1) * 4 <= 160 * 1024, "LDS budget");
static_assert(kRoundPages <= kPagesPerThread * kThreads && kRoundPages <= 1024 && kRoundReqs <= 8,
              "round page fields");
static_assert(kQPiecesPerThread * kThreads == kRoundReqs * kTileRows * 16, "query pieces");
static_assert(IDX_SCORE_SORT_BUCKETS <= kTileRows * kRoundPages, "the bucket histogram fits the stage");


// Fill the round's LDS (all threads; one barrier inside).  Pages [lo, lo + np)
// of the step belong to requests r0 .. r0 + nreq - 1.
template <int FMT>
__device__ void setup_round(const StepArgs& a, RoundLds& L, const uint32_t* pre, const int32_t* slot_of, int r0,
                            int nreq, uint32_t lo, int np, int tid) {
  const int P = a.P, H = a.H, rows = P * H, MB = a.max_blocks;
  if (tid < nreq) {
    const int r = r0 + tid;
    RoundReq& rq = L.req[tid];
    rq.r = r;
    rq.p0 = (int)pre[r];
    rq.nbg = (int)(pre[r + 1] - pre[r]);
    int lm = INT_MAX;
    int lv[kTileRows];  // P <= 16: every load issues before any is used
#pragma unroll
    for (int j = 0; j < kTileRows; ++j) lv[j] = a.row_len[r * P + min(j, P - 1)];
#pragma unroll
    for (int j = 0; j < kTileRows; ++j) lm = min(lm, clamp_len(lv[j], MB));  // repeats of row P - 1 change nothing
    rq.lmin = lm;
    rq.sigma = 0;
    L.amax[tid] = 0;
  }
  if (tid < nreq * kTileRows) {
    const int j = tid / kTileRows, i = tid % kTileRows;
    L.req[j].len[i] = (i < rows) ? clamp_len(a.row_len[(r0 + j) * P + i / H], MB) : 0;
  }
  int pk[kPagesPerThread], jk[kPagesPerThread];
#pragma unroll
  for (int m = 0; m < kPagesPerThread; ++m) {
    const int k = tid + kThreads * m;
    pk[m] = -1;
    jk[m] = 0;
    if (k < np) {
      const uint32_t u = lo + (uint32_t)k;
      int j = 0;
      while (j + 1 < nreq && pre[r0 + j + 1] <= u) ++j;
      const int r = r0 + j;
      const int slot = slot_of[r];  // a request with pages is no graph pad
      pk[m] = a.block_table[(int64_t)slot * MB + (int)(u - pre[r])];
      jk[m] = j;
      L.ridx[k] = (uint8_t)j;
    }
  }
  // query tiles (loaded before the page order is sorted, so their latency
  // overlaps it): piece e = (request j, row, group of 8 values); kQPiecesPerThread per thread
  u32x4 pc[kQPiecesPerThread];
#pragma unroll
  for (int i = 0; i < kQPiecesPerThread; ++i) {
    const int e = tid + kThreads * i, j = e >> 8, row = (e >> 4) & 15, col = (e & 15) * 8;
    pc[i] = u32x4{0u, 0u, 0u, 0u};
    if (j < nreq && row < rows)
      pc[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                              ((int64_t)(r0 + j) * rows + row) * kHeadDim + col);
  }
  int pos[kPagesPerThread];  // hand-out position of each page
#pragma unroll
  for (int m = 0; m < kPagesPerThread; ++m) pos[m] = tid + kThreads * m;
#if IDX_SCORE_SORT_BUCKETS > 0
  if (np >= IDX_SCORE_SORT_MIN) {
    // by page id: a counting sort into NB equal buckets of the pool, so that
    // all workgroups sweep the pool from its low pages to its high ones
    // together
    constexpr int NB = IDX_SCORE_SORT_BUCKETS;
    uint32_t* hist = reinterpret_cast<uint32_t*>(&L.stage[0][0]);
    for (int b = tid; b < NB; b += kThreads) hist[b] = 0;
    __syncthreads();
    int bk[kPagesPerThread];
    uint32_t rank[kPagesPerThread];
#pragma unroll
    for (int m = 0; m < kPagesPerThread; ++m) {
      rank[m] = 0;
      const int k = tid + kThreads * m;
      const int pid = pk[m];
      bk[m] = (pid >= 0 && pid < a.n_pages) ? (int)((uint64_t)pid * NB / (uint64_t)a.n_pages) : NB - 1;
      if (k < np) rank[m] = atomicAdd(&hist[bk[m]], 1u);
    }
    __syncthreads();
    constexpr int PER = (NB + kThreads - 1) / kThreads;  // bins a thread scans
    uint32_t h[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      h[i] = (PER * tid + i < NB) ? hist[PER * tid + i] : 0u;
      sum += h[i];
    }
    uint32_t tot;
    uint32_t start = block_exclusive_scan<kThreads>(sum, L.wave_tot, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (PER * tid + i < NB) hist[PER * tid + i] = start;
      start += h[i];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kPagesPerThread; ++m) pos[m] = (int)(hist[bk[m]] + rank[m]);
  }
#endif
#pragma unroll
  for (int m = 0; m < kPagesPerThread; ++m) {
    const int k = tid + kThreads * m;
    if (k < np) {
      L.pid[pos[m]] = pk[m];
      L.sk[pos[m]] = (uint16_t)(k | (jk[m] << 10));
    }
  }
  if constexpr (FMT == IDX_K_NVFP4) {
    __syncthreads();  // amax cleared
#pragma unroll
    for (int i = 0; i < kQPiecesPerThread; ++i) {
      const int e = tid + kThreads * i, j = e >> 8;
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(pc[i][w] << 16)), fabsf(__uint_as_float(pc[i][w] & 0xFFFF0000u))));
      if (j < nreq) atomicMax(&L.amax[j], __float_as_uint(m));  // non-negative floats order as integers
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQPiecesPerThread; ++i) {
      const int e = tid + kThreads * i, j = e >> 8;
      if (j >= nreq) continue;
      const float amax = __uint_as_float(L.amax[j]);
      int sigma = 0;
      if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);  // amax < 2^ex
        sigma = 15 - ex;
      }
      if ((e & 255) == 0) L.req[j].sigma = sigma;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const _Float16 lo16 = (_Float16)ldexpf(__uint_as_float(pc[i][w] << 16), sigma);
        const _Float16 hi16 = (_Float16)ldexpf(__uint_as_float(pc[i][w] & 0xFFFF0000u), sigma);
        pc[i][w] = (uint32_t)__builtin_bit_cast(uint16_t, lo16) | ((uint32_t)__builtin_bit_cast(uint16_t, hi16) << 16);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kQPiecesPerThread; ++i) {
    const int e = tid + kThreads * i, j = e >> 8, row = (e >> 4) & 15, col = (e & 15) * 8;
    if (j < nreq) *reinterpret_cast<u32x4*>(&L.q[j][row][col]) = pc[i];
  }
  if (tid == 0) L.next = 0;
}

// Fused store of a step's new NVFP4 keys (st_n of them, at most
// IDX_FP4_FUSED_MAX_KEYS): the same bytes idx_fp4_store writes, eight lanes a
// key.  Every key is written twice over: by workgroup t mod G (wave 1, while
// the other waves stream), so that keys in pages no workgroup reads reach the
// pool too, and by wave 0 of each workgroup whose round holds the key's page,
// before any wave of that workgroup reads the page.  Both write identical
// bytes, so their order does not matter; the reading wave sees wave 0's
// write through its own CU's caches once wave 0's stores are complete, which
// wave 0 publishes in LDS.  No workgroup waits for another.
__device__ __forceinline__ void store_new_key(const StepArgs& a, int64_t t, int grp, int64_t n_slots) {
  const u32x4* src = reinterpret_cast<const u32x4*>(a.st_staging + t * a.st_stride + 16 * grp);
  const u32x4 w0 = src[0], w1 = src[1];
  const int64_t slot = a.st_slots[t];
  if (slot < 0 || slot >= n_slots) return;  // the key's eight lanes skip it together
  quantize_group(w0, w1, slot, grp, const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.k)),
                 const_cast<uint8_t*>(a.k_scale));
}

// The keys whose page this round reads (np pages in L.pid; when the round
// was sorted, the first NB words of the stage hold each bucket's first
// position), found per key in its bucket's range from the slots each thread
// loaded at the start: listed for wave 0 to store, and their pages marked in
// sk, so that a wave handed such a page waits until wave 0 has stored them.
__device__ void mark_round_keys(const StepArgs& a, RoundLds& L, int np, int tid, const int64_t* kslot) {
  constexpr int NB = IDX_SCORE_SORT_BUCKETS;
  const uint32_t* starts = reinterpret_cast<const uint32_t*>(&L.stage[0][0]);
  const int64_t n_slots = a.n_pages * kBlock;
  const bool sorted = NB > 0 && np >= IDX_SCORE_SORT_MIN;
  if (tid == 0) {
    L.n_own = 0u;
    L.keys_ready = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int64_t slot = kslot[i];
    if (slot < 0 || slot >= n_slots) continue;  // past the keys, or a slot the store skips
    const int page = (int)(slot / kBlock);
    int k0 = 0, k1 = np;
    if (sorted) {
      const int bk = (int)((uint64_t)page * (uint64_t)(NB > 0 ? NB : 1) / (uint64_t)a.n_pages);
      k0 = (int)starts[bk];
      k1 = bk + 1 < NB ? (int)starts[bk + 1] : np;
    }
    bool found = false;
    for (int k = k0; k < k1; ++k)
      if (L.pid[k] == page) {
        // keys of one page set the same bit: concurrent writes agree
        L.sk[k] = (uint16_t)(L.sk[k] | kSkNewKeys);
        found = true;
      }
    if (found) L.own[atomicAdd(&L.n_own, 1u)] = (uint16_t)(tid + kThreads * i);
  }
  __syncthreads();
}

// A wave handed a round page that holds new keys waits until wave 0 has
// stored them (wave 0 stores them before it takes any page, so it never
// waits itself; the bound only keeps the loop finite).
__device__ __forceinline__ void wait_round_keys(RoundLds& L) {
  for (int it = 0; it < (1 << 24); ++it) {
    if (__hip_atomic_load(&L.keys_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) return;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Keys b, b + G, ... (this workgroup's share of the writes that also cover
// keys in pages no workgroup reads), eight lanes a key, from `lanes` lanes.
__device__ __forceinline__ void store_cyclic_keys(const StepArgs& a, int lane, int lanes) {
  const int64_t n_slots = a.n_pages * kBlock;
  for (int64_t t = blockIdx.x + (int64_t)gridDim.x * (lane >> 3); t < a.st_n; t += (int64_t)gridDim.x * (lanes >> 3))
    store_new_key(a, t, lane & 7, n_slots);
}

// One wave's part of a round: pages from the round's counter until none is
// left.  Wave page p (two units) is described by lane p % 64 of vm_tag (round
// page | request << 16, or -1) and vm_pid.
template <int FMT, int MODE, bool KEYS>
__device__ __forceinline__ void stream_round(const StepArgs& a, RoundLds& L, uint32_t lo, int np, int lane,
                                             int n, int g, int wave, bool first) {
  typedef typename Fmt<FMT>::Op Op;
  constexpr int kRing = Fmt<FMT>::kRing;
  static_assert(kRing >= 2, "at least one half page in flight");
  constexpr int kPageBytes = kBlock * Fmt<FMT>::kRowBytes;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* ks = a.k_scale;
  const int rows = a.P * a.H;
  const int wrow = 4 * g + n;  // lanes n < 4 hold row 4g + n
  const bool writer = n < 4 && wrow < rows;

  int vm_tag = -1, vm_pid = -1;
  bool done = false;
  int last = -1;  // last wave page that holds a page

  int cur = -1, p0 = 0, lmin = 0, sigma = 0, my_len = 0;
  float c2 = 0.f;  // lse: sm_scale * log2 e * 2^-sigma
  int len[4] = {0, 0, 0, 0};
  Op qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = Op{};
  float st0[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float st1[4] = {0.f, 0.f, 0.f, 0.f};

  if constexpr (KEYS) {
    // the fused store: wave 0 writes the keys of this round's pages before it
    // takes a page, wave 1 its share of all keys in the first round
    {
      if (wave == 0) {
        const int64_t n_slots = a.n_pages * kBlock;
        const int no = (int)uniform(L.n_own);
        for (int i = lane >> 3; i < no; i += 8) store_new_key(a, L.own[i], lane & 7, n_slots);
        __builtin_amdgcn_s_waitcnt(0);  // wave 0's stores are complete
        if (lane == 0) __hip_atomic_store(&L.keys_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else if (wave == 1 && first) {
        store_cyclic_keys(a, lane, 64);
      }
    }
  }

  auto issue = [&](Half<FMT>& h, int V) {
    const int p = V >> 1;
    if ((V & 1) == 0) {
      int tag = -1, pid = -1;
      if (!done) {
        uint32_t k = 0;
        if (lane == 0) k = atomicAdd(&L.next, 1u);
        k = uniform(k);
        if (k < (uint32_t)np) {
          pid = (int)uniform((uint32_t)L.pid[k]);
          const uint32_t skv = uniform((uint32_t)L.sk[k]);
          if constexpr (KEYS) {
            if (skv & kSkNewKeys) wait_round_keys(L);  // the page holds new keys
          }
          tag = (int)((skv & 1023u) | (((skv >> 10) & 7u) << 16));
          last = p;
        } else {
          done = true;
        }
      }
      if (lane == (p & 63)) {
        vm_tag = tag;
        vm_pid = pid;
      }
    }
    const int tag = __builtin_amdgcn_readlane(vm_tag, p & 63);
    const int pid = __builtin_amdgcn_readlane(vm_pid, p & 63);
    const bool ok = tag >= 0 && pid >= 0 && pid < a.n_pages;
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(kp, pid, ok, kPageBytes);
    const __amdgpu_buffer_rsrc_t rs = (FMT == IDX_K_NVFP4) ? page_rsrc(ks, pid, ok, kBlock * 8) : rk;
    load_half<FMT>(h, rk, rs, V & 1, n, g);
  };

  auto compute = [&](const Half<FMT>& h, int U) {
    const int p = U >> 1;
    const int tag = __builtin_amdgcn_readlane(vm_tag, p & 63);
    if (tag < 0) return;
    const int k = tag & 0xFFFF, j = tag >> 16;
    if ((U & 1) == 0) {
      if (j != cur) {  // another request: its context from the round
        cur = j;
        const RoundReq& rq = L.req[j];
        p0 = (int)uniform((uint32_t)rq.p0);
        lmin = (int)uniform((uint32_t)rq.lmin);
        sigma = (int)uniform((uint32_t)rq.sigma);
        if constexpr (MODE == IDX_SCORE_LSE) c2 = ldexpf(a.sm_scale * 1.44269504088896341f, -sigma);
        const u32x4 lv = *reinterpret_cast<const u32x4*>(&rq.len[4 * g]);
        len[0] = (int)lv.x; len[1] = (int)lv.y; len[2] = (int)lv.z; len[3] = (int)lv.w;
        my_len = (n == 0) ? len[0] : (n == 1) ? len[1] : (n == 2) ? len[2] : len[3];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          qf[s] = __builtin_bit_cast(Op, *reinterpret_cast<const u32x4*>(&L.q[j][n][Fmt<FMT>::d0(s, g)]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st0[e] = -INFINITY;
        st1[e] = 0.f;
      }
    }
    const int b = (int)(lo + (uint32_t)k) - p0;
    const bool full = (b + 1) * kBlock <= lmin;
    score_half<FMT, MODE>(h, qf, full, b * kBlock + 64 * (U & 1) + n, len, st0, st1, c2);
    if (U & 1) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float m = row16_max(st0[e]);
        if constexpr (MODE == IDX_SCORE_MAX) {
          v[e] = m;
        } else {
          // the 16 lanes' sums rescaled to the block's max, then ln = log2 * ln 2
          const float base = (m == -INFINITY) ? 0.f : m;
          const float sum = row16_sum(st1[e] * __builtin_amdgcn_exp2f(st0[e] - base));
          v[e] = (m == -INFINITY) ? -INFINITY : (m + __builtin_amdgcn_logf(sum)) * 0.693147180559945309f;
        }
      }
      float o = (n == 0) ? v[0] : (n == 1) ? v[1] : (n == 2) ? v[2] : v[3];
      if constexpr (FMT == IDX_K_NVFP4 && MODE == IDX_SCORE_MAX) o = ldexpf(o, -sigma);
      const int pid = __builtin_amdgcn_readlane(vm_pid, p & 63);
      if (!(pid >= 0 && pid < a.n_pages)) o = (b * kBlock < my_len) ? __builtin_nanf("") : -INFINITY;
      if (writer) L.stage[wrow][k] = o;
    }
  };

  // a trip covers an even number of units, so ring slots and halves are static
  constexpr int kTrip = (kRing % 2) ? 2 * kRing : kRing;
  Half<FMT> ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) issue(ring[u], u);
  for (int U0 = 0;; U0 += kTrip) {
#pragma unroll
    for (int k = 0; k < kTrip; ++k) {
      issue(ring[(k + kRing - 1) % kRing], U0 + k + kRing - 1);
      compute(ring[k % kRing], U0 + k);
    }
    if (done && 2 * (last + 1) <= U0 + kTrip) break;  // every held page is computed
  }
}

// The round's block scores to their rows (all threads): runs of consecutive
// blocks per row and request.
__device__ __forceinline__ void write_round(const StepArgs& a, const RoundLds& L, uint32_t lo, int np, int tid) {
  const int rows = a.P * a.H, MB = a.max_blocks;
  for (int i = 0; i < rows; ++i)
    for (int k = tid; k < np; k += kThreads) {
      const RoundReq& rq = L.req[L.ridx[k]];
      const int b = (int)(lo + (uint32_t)k) - rq.p0;
#if IDX_SCORE_NT_OUT
      __builtin_nontemporal_store(L.stage[i][k], &a.block_scores[((int64_t)rq.r * rows + i) * MB + b]);
#else
      a.block_scores[((int64_t)rq.r * rows + i) * MB + b] = L.stage[i][k];
#endif
    }
}

// The request holding step page x: the largest r < R with pre[r] <= x, in
// every lane of the wave (pre[0] = 0 <= x).  Each pass checks 64 evenly
// spaced candidates with one LDS read per lane.
__device__ __forceinline__ int request_of(const uint32_t* pre, int R, uint32_t x, int lane) {
  int lo = 0, hi = R;  // the answer lies in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) >> 6;
    const int r = lo + step * lane;
    const int below = __popcll(__ballot(r < hi && pre[min(r, R)] <= x));  // a prefix of the lanes, lane 0 included
    lo += step * (below - 1);
    hi = min(hi, lo + step);
  }
  return lo;
}

// Each workgroup's page rate on its last launch (pages a 10 ns tick, 2^16
// fixed point; 0: none yet), per device.  Workgroup b runs on XCD b % 8; the
// next launch sizes each XCD's shares in proportion to its workgroups' summed
// rates.  Calls racing on it change only how the pages are shared, never a
// result.
__device__ uint32_t g_wg_rate[1024];

template <int FMT, int MODE, bool KEYS>
__global__ __launch_bounds__(kThreads) void score_kernel(const StepArgs a) {
  static_assert(!KEYS || FMT == IDX_K_NVFP4, "the fused store is for NVFP4 keys");
  extern __shared__ uint32_t pre[];  // n_req + 1 prefix sums of per-request block counts, then n_req slots
  __shared__ RoundLds L;
  __shared__ uint32_t wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int P = a.P, rows = P * a.H, MB = a.max_blocks, R = a.n_req;
  int32_t* slot_of = reinterpret_cast<int32_t*>(pre + R + 1);

  // 0. NVFP4 with new keys: their slots, loaded now for the rounds' lookups
  int64_t kslot[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) kslot[i] = -1;
  if constexpr (KEYS) {
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i)
      if (tid + kThreads * i < a.st_n) kslot[i] = a.st_slots[tid + kThreads * i];
  }

  // 1. pages each request's group reads (0 for graph pads) and their prefix
  // sums; the slots stay in LDS for the rounds
  uint32_t carry = 0;
  for (int base = 0; base < R; base += kThreads) {
    const int r = base + tid;
    uint32_t nbg = 0;
    if (r < R) {
      const int slot = a.req_slot[r];
      int lmax = 0;  // loaded without waiting for the slot
      int lv[kTileRows];  // P <= 16: every load issues before any is used
#pragma unroll
      for (int j = 0; j < kTileRows; ++j) lv[j] = a.row_len[r * P + min(j, P - 1)];
#pragma unroll
      for (int j = 0; j < kTileRows; ++j) lmax = max(lmax, clamp_len(lv[j], MB));  // repeats change nothing
      slot_of[r] = slot;
      if (slot >= 0 && slot < a.n_slot_rows) nbg = (uint32_t)blocks_of(lmax);
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kThreads>(nbg, wave_tot, &tot);
    if (r < R) pre[r] = carry + ex;
    carry += tot;
  }
  if (tid == 0) pre[R] = carry;
  __syncthreads();
  const uint32_t N = uniform(carry);

  // 2. this workgroup's share of the step's pages, in rounds: equal, or in
  // proportion to its XCD's measured rate
  const int G = gridDim.x, b = blockIdx.x;
  uint32_t lo = (uint32_t)((uint64_t)b * N / G);
  uint32_t hi = (uint32_t)((uint64_t)(b + 1) * N / G);
  constexpr uint64_t kPageKBytes = (uint64_t)kBlock * (Fmt<FMT>::kRowBytes + (FMT == IDX_K_NVFP4 ? 8 : 0));
  const bool adapt = IDX_SCORE_ADAPT && (G % 8) == 0 && G <= 1024 &&
                     (uint64_t)N * kPageKBytes >= (uint64_t)IDX_SCORE_ADAPT_MIN_BYTES * G;
  if (adapt) {
    uint32_t* xs = reinterpret_cast<uint32_t*>(&L.stage[0][0]);  // [0, 8): summed rates, [8, 16): known
    if (tid < 16) xs[tid] = 0;
    __syncthreads();
    for (int w = tid; w < G; w += kThreads) {
      const uint32_t v = g_wg_rate[w];
      atomicAdd(&xs[w & 7], v);
      atomicAdd(&xs[8 + (w & 7)], v != 0u ? 1u : 0u);
    }
    __syncthreads();
    uint64_t wx[8], w8 = 0;
    bool known = true;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      wx[x] = uniform(xs[x]);
      known = known && uniform(xs[8 + x]) == (uint32_t)(G / 8);
      w8 += wx[x];
    }
    __syncthreads();  // the stage is the round's again
    if (known && w8 > 0) {
      auto cum = [&](int c) -> uint64_t {  // weight of workgroups 0 .. c - 1
        uint64_t t = (uint64_t)(c / 8) * w8;
#pragma unroll
        for (int x = 0; x < 8; ++x) t += (x < (c & 7)) ? wx[x] : 0u;
        return t;
      };
      const uint64_t total = (uint64_t)(G / 8) * w8;
      lo = (uint32_t)((uint64_t)N * cum(b) / total);
      hi = (uint32_t)((uint64_t)N * cum(b + 1) / total);
    }
  }
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  if (a.n_pages == 0) {
    // nothing can be read: every visible block is NaN
    for (uint32_t u = lo + tid; u < hi; u += kThreads) {
      int rlo = 0, rhi = R;
      while (rhi - rlo > 1) {
        const int mid = (rlo + rhi) >> 1;
        if (pre[mid] <= u) rlo = mid; else rhi = mid;
      }
      const int b = (int)(u - pre[rlo]);
      for (int i = 0; i < rows; ++i) {
        const int L0 = clamp_len(a.row_len[rlo * P + i / a.H], MB);
        a.block_scores[((int64_t)rlo * rows + i) * MB + b] = (b * kBlock < L0) ? __builtin_nanf("") : -INFINITY;
      }
    }
  } else {
    for (uint32_t rl = lo; rl < hi;) {
      const int r0 = request_of(pre, R, rl, lane);  // pre[r0] <= rl < pre[r0 + 1]
      const int rend = min(R, r0 + kRoundReqs);
      const uint32_t rh = min(min(hi, rl + (uint32_t)kRoundPages), uniform(pre[rend]));
      // requests r0 .. rend - 1 that start before rh (a prefix: pre does not decrease)
      const bool starts = lane < rend - r0 && pre[min(r0 + lane, R)] < rh;
      const int nreq = __popcll(__ballot(starts));
      const int np = (int)(rh - rl);
      setup_round<FMT>(a, L, pre, slot_of, r0, nreq, rl, np, tid);
      __syncthreads();
      if constexpr (KEYS) mark_round_keys(a, L, np, tid, kslot);
      stream_round<FMT, MODE, KEYS>(a, L, rl, np, lane, n, g, wave, rl == lo);
      __syncthreads();
      write_round(a, L, rl, np, tid);
      __syncthreads();
      rl = rh;
    }
  }
  if constexpr (KEYS) {
    // a workgroup that streamed nothing still writes its share of the keys
    if (lo >= hi || a.n_pages == 0) store_cyclic_keys(a, tid, kThreads);
  }

  if (adapt) {
    const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t_start;
    // below 2^20, so that N (< 2^26 pages) times the summed weights stays in 64 bits
    const uint32_t rate = (uint32_t)min((uint64_t)(hi - lo) * 65536u / (dt > 0 ? dt : 1), (uint64_t)0xFFFFF);
    if (tid == 0 && hi > lo) {
      const uint32_t old = g_wg_rate[b];
      g_wg_rate[b] = old ? (old + rate) / 2 : rate;
    }
  }

  // 3. -inf past each group's extent, and everywhere for graph pads: one
  // output row per workgroup in turn, after the rounds so that the first K
  // loads do not wait for it
  for (int q = blockIdx.x; q < R * rows; q += gridDim.x) {
    const int r = q / rows;
    const int nbg = (int)(uniform(pre[r + 1]) - uniform(pre[r]));
    float* out = a.block_scores + (int64_t)q * MB;
    for (int c = nbg + tid; c < MB; c += kThreads) out[c] = -INFINITY;
  }
  (void)wave;
}

namespace {
size_t dyn_bytes(int n_req) { return (size_t)(2 * n_req + 1) * sizeof(uint32_t); }

// Workgroups that fit on the device at once (cached per device), with the
// dynamic LDS limit raised to what the largest request count needs.
template <int FMT, int MODE, bool KEYS>
int resident_workgroups() {
  static std::atomic<int> cache[64];  // zero-initialised; calls from several threads store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int n = cache[dev].load(std::memory_order_relaxed); n > 0) return n;
  const size_t smem = dyn_bytes(IDX_MAX_REQ);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(score_kernel<FMT, MODE, KEYS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(score_kernel<FMT, MODE, KEYS>),
                                                   kThreads, smem) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev].store(cus * per_cu, std::memory_order_relaxed);
  return cus * per_cu;
}

template <int FMT, int MODE, bool KEYS = false>
void launch(const StepArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((score_kernel<FMT, MODE, KEYS>), dim3(resident_workgroups<FMT, MODE, KEYS>()), dim3(kThreads),
                     dyn_bytes(a.n_req), stream, a);
}

template <int MODE>
void launch_mode(const StepArgs& a, hipStream_t stream) {
  switch (a.k_format) {
    case IDX_K_BF16: launch<IDX_K_BF16, MODE>(a, stream); break;
    case IDX_K_FP8_E4M3: launch<IDX_K_FP8_E4M3, MODE>(a, stream); break;
    default:  // NVFP4: the kernel with the fused store only when there are new keys
      if (a.st_n > 0)
        launch<IDX_K_NVFP4, MODE, true>(a, stream);
      else
        launch<IDX_K_NVFP4, MODE>(a, stream);
      break;
  }
}
}  // namespace

hipError_t launch_score(const StepArgs& a, hipStream_t stream) {
  if (a.n_req == 0 || a.max_blocks == 0) return hipSuccess;
  if (a.P * a.H > kTileRows) return launch_score_rows(a, stream);
  if (a.score_mode == IDX_SCORE_LSE)
    launch_mode<IDX_SCORE_LSE>(a, stream);
  else
    launch_mode<IDX_SCORE_MAX>(a, stream);
  return hipGetLastError();
}

}  // namespace idx
