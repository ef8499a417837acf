// topk.hip -- forced block top-k per (row, head) for gfx950.
//
// Selection (sglang PR 42614, Modifications item 1 and Accuracy Tests): with
// nb = ceil(row_len / 128) blocks, every block is taken when nb <= topk;
// otherwise the first init_blocks and the last local_blocks of the row's own
// nb are always taken and the remaining topk - |forced| slots go to the
// highest block scores, ties to the lower block id.  Selection is exact.
//
// One workgroup of NT threads per (row, head): for rows of at most 2,048
// blocks, 512 threads of up to 4 blocks when there are at most 512 rows (the
// launch is then one row's latency, which more threads shorten: 256 rows of
// 1,024 blocks 7.3 against 7.9 us), else 256 (1,024 rows of 1,184 blocks: 7.5
// against 9.4 us with 512); wider rows 512 (560 rows of 4,096: 9.8 against
// 9.2 us with 256).  Thread t owns the contiguous blocks
// [t*C, t*C + C), C = ceil(max_blocks / NT) <= 4, 8 or 16 (rounded up to
// a multiple of 4 when rows are 16-byte aligned), and loads their scores into
// registers first thing; the row's slot and length are fetched before them and
// the score loads do not wait for them.  Keys are 32-bit integers whose
// unsigned order is the selection order: NaN below every number, -0 equal to
// +0; each thread computes its keys once and marks its competing and forced
// blocks in two bit masks.  A radix select over the competing keys finds the
// k-th largest key T, k = topk - |forced|: it starts at the highest bit where
// those keys differ, takes up to 11 bits a pass into a 2,048-bin LDS histogram
// (thread t scans and clears 2,048 / NT bins), and stops once the chosen bin holds
// exactly the keys still needed.  One packed scan of (taken-for-sure,
// equal-to-T) counts then gives every thread its output positions, so ids
// leave in ascending order without a sort.  Reductions and scans inside a
// wave use DPP; waves meet through LDS.
//
// Many short rows (at least 1,024 rows of at most 1,024 blocks, as prefill
// gives, or rows of at most 64 blocks) take one wave a row and no workgroup
// barrier instead: lane l holds blocks l, l + 64, ...; T is found by a radix
// select over 8-bit digits with a 256-bin LDS histogram of the wave's own
// (IDX_TOPK_RADIX 1; bit by bit with one wave-wide count a bit measured
// slower, 33.3 against 28.4 us on 32,768 rows of 272 blocks), stopping once
// the chosen bin holds exactly the keys still needed; ties and output
// positions come from ballot masks.
#include "device.h"


#ifndef IDX_TOPK_VALU_COUNT
#define IDX_TOPK_VALU_COUNT 1  // bit-by-bit one-wave kernel: 1 counts keys per lane and sums them with
#endif                         // DPP (vector work); 0: a ballot and a scalar popcount per slot
#ifndef IDX_TOPK_RADIX
#define IDX_TOPK_RADIX 1           // one-wave kernel: 1 finds its threshold by 8-bit digits over LDS
#endif                             // histograms; 0: bit by bit, one wave-wide count a bit
#ifndef IDX_TOPK_BALLOT_BUFLOAD
#define IDX_TOPK_BALLOT_BUFLOAD 1  // one-wave kernel: score loads through a row descriptor (no branches)
#endif
#ifndef IDX_TOPK_BALLOT_SCHED
#define IDX_TOPK_BALLOT_SCHED 1  // one-wave kernel: slot and length loads issue before the score loads
#endif
#ifndef IDX_TOPK_WIDE_ROWS
#define IDX_TOPK_WIDE_ROWS 512  // up to this many rows of <= 2,048 blocks: 512 threads of 4 blocks a row
#endif                          // (256 rows of 1,024: 7.9 -> 7.3 us); more rows keep 256 threads of 8
#ifndef IDX_TOPK_BALLOT_ROWS
#define IDX_TOPK_BALLOT_ROWS 1024  // rows from which rows of <= 1,024 blocks take one wave each
#endif

namespace idx {

constexpr int kTopkThreads = 512;        // the workgroup kernel: one row a workgroup
constexpr int kTopkThreadsNarrow = 256;  // its threads for rows of at most 2,048 blocks
#ifndef IDX_TOPK_BALLOT_THREADS
#define IDX_TOPK_BALLOT_THREADS 256  // the one-wave kernel's workgroup: a row a wave
#endif
constexpr int kBallotThreads = IDX_TOPK_BALLOT_THREADS;
constexpr int kBallotWaves = kBallotThreads / 64;

#ifndef IDX_TOPK_KEY_ADD0
#define IDX_TOPK_KEY_ADD0 1  // order keys: -0 made +0 by adding +0 (fewer vector instructions)
#endif
__device__ __forceinline__ uint32_t order_key(float f) {
#if IDX_TOPK_KEY_ADD0
  // f + 0 is f except that -0 becomes +0 (round to nearest); negative
  // values flip every bit, others set the sign bit; NaN ranks lowest
  const uint32_t u = __float_as_uint(f + 0.0f);
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return (f == f) ? k : 0u;
#else
  if (f != f) return 0u;  // NaN
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
#endif
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum across the 64 lanes of a wave (row_shr within rows of
// 16 lanes, then row_bcast:15 / row_bcast:31 across rows).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += dpp_u32<0x111>(x);        // row_shr:1
  x += dpp_u32<0x112>(x);        // row_shr:2
  x += dpp_u32<0x114>(x);        // row_shr:4
  x += dpp_u32<0x118>(x);        // row_shr:8
  x += dpp_u32<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_u32<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Exclusive prefix sum over the workgroup; *total gets the sum of all.  One
// barrier: the caller must not reuse `wave_tot` before another barrier.
template <int NW>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wave_tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  *total = all;
  return before + incl - v;
}

// Within each row of 16 lanes every lane gets the row's min / max / sum
// (quad_perm and row_ror patterns keep every lane's source valid).
template <int OP>
__device__ __forceinline__ uint32_t combine(uint32_t a, uint32_t b) {
  return OP == 0 ? min(a, b) : OP == 1 ? max(a, b) : a + b;
}
template <int OP>
__device__ __forceinline__ uint32_t row16_reduce(uint32_t x) {
  x = combine<OP>(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = combine<OP>(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = combine<OP>(x, dpp_u32<0x124>(x));  // row_ror:4
  x = combine<OP>(x, dpp_u32<0x128>(x));  // row_ror:8
  return x;
}

// Whole-wave reduction (0 min, 1 max, 2 sum), returned wave-uniform.
template <int OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  x = row16_reduce<OP>(x);
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return combine<OP>(combine<OP>(a, b), combine<OP>(c, d));
}

// PER: blocks per thread, NT threads (8 x 256 covers max_blocks <= 2048, 8 x 512
// <= 4096, 16 x 512 the full limit).
template <int PER, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(const StepArgs a) {
  constexpr int kTopkWaves = NT / 64;
  static_assert(PER <= 32, "per-thread block sets are 32-bit masks");
  constexpr int kBins = 2048, kBinsPerThread = kBins / NT;  // 4 or 8
  __shared__ u32x4 hist4[kBins / 4];
  uint32_t* hist = reinterpret_cast<uint32_t*>(hist4);
  __shared__ uint32_t red[3][kTopkWaves];
  __shared__ uint32_t wave_tot[2][kTopkWaves];
  __shared__ uint32_t pick_digit, pick_above, pick_count;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = a.P * a.H;
  const int o = blockIdx.x;
  const int r = o / rows, i = o - r * rows;
  const int K = a.topk, MB = a.max_blocks;
  const float* bs = a.block_scores + (int64_t)o * MB;

  // the row's slot and length first: these two scalar loads must not queue
  // behind the burst of score loads below
  const int slot = a.req_slot[r];
  const int len_raw = a.row_len[r * a.P + i / a.H];
  __builtin_amdgcn_sched_barrier(0);

  // this thread's scores (they do not wait for the length); 16-byte loads
  // when every thread's range starts 16-byte aligned
  const bool vec = (MB % 4) == 0 && (reinterpret_cast<uintptr_t>(a.block_scores) & 15u) == 0;
  const int C = vec ? ((MB / 4 + NT - 1) / NT) * 4 : (MB + NT - 1) / NT;
  const int b0 = tid * C;
  float sv[PER];
  if (vec) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      f32x4 v = (4 * q < C && b0 + 4 * q < MB) ? *reinterpret_cast<const f32x4*>(bs + b0 + 4 * q)
                                               : f32x4{0.f, 0.f, 0.f, 0.f};
      sv[4 * q] = v[0]; sv[4 * q + 1] = v[1]; sv[4 * q + 2] = v[2]; sv[4 * q + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) sv[j] = (j < C && b0 + j < MB) ? bs[b0 + j] : 0.0f;
  }

  // this thread's bins, highest digits first: [kBins - B(t+1), kBins - B t), B = kBinsPerThread
  const int bin0 = kBins - kBinsPerThread * (tid + 1);
#pragma unroll
  for (int q = 0; q < kBinsPerThread / 4; ++q) hist4[bin0 / 4 + q] = u32x4{0u, 0u, 0u, 0u};

  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  const int nb = pad ? 0 : blocks_of(clamp_len(len_raw, MB));
  int32_t* ids = a.topk_ids + (int64_t)o * K;
  float* sc = a.topk_scores + (int64_t)o * K;

  if (nb <= K) {
    for (int t = tid; t < K; t += NT) {
      ids[t] = t < nb ? t : -1;
      sc[t] = t < nb ? bs[t] : -INFINITY;
    }
    return;
  }

  // keys once; bit j of `cand` marks a block that competes, of `forced` one
  // that is always taken
  const int cnt = max(0, min(C, nb - b0));
  const int init = a.init_blocks, local_from = nb - a.local_blocks;
  uint32_t key[PER];
  uint32_t cand = 0, forced = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = b0 + j;
    const bool is_forced = b < init || b >= local_from;
    key[j] = order_key(sv[j]);
    if (j < cnt) {
      if (is_forced) {
        forced |= 1u << j;
      } else {
        cand |= 1u << j;
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
    }
  }
  kmin = wave_reduce<0>(kmin);
  kmax = wave_reduce<1>(kmax);
  const uint32_t nforced = wave_reduce<2>((uint32_t)__builtin_popcount(forced));
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
    red[2][wave] = nforced;
  }
  __syncthreads();
  uint32_t F = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    kmin = min(kmin, red[0][w]);
    kmax = max(kmax, red[1][w]);
    F += red[2][w];
  }

  // radix select of the want-th largest competing key
  uint32_t want = (uint32_t)K - F;  // the free slots (F <= init + local <= K)
  uint32_t prefix = kmin, tshift = 0;
  if (want > 0 && kmin != kmax) {
    int hi = 31 - __builtin_clz(kmin ^ kmax);
    prefix = (hi == 31) ? 0u : (kmin >> (hi + 1)) << (hi + 1);
    while (hi >= 0) {
      const int lo = max(hi - 10, 0);
      const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const bool match = (hi == 31) || ((key[j] >> (hi + 1)) == (prefix >> (hi + 1)));
        if (((cand >> j) & 1u) && match) atomicAdd(&hist[(key[j] >> lo) & dmask], 1u);
      }
      __syncthreads();
      // this thread's bins (descending digits) into registers, then clear them
      uint32_t h[kBinsPerThread];
#pragma unroll
      for (int q = 0; q < kBinsPerThread / 4; ++q) {
        const u32x4 v = hist4[bin0 / 4 + q];
        h[4 * q] = v[0]; h[4 * q + 1] = v[1]; h[4 * q + 2] = v[2]; h[4 * q + 3] = v[3];
      }
      uint32_t local = 0;
#pragma unroll
      for (int q = 0; q < kBinsPerThread; ++q) local += h[q];
      uint32_t tot;
      const uint32_t above = block_scan<kTopkWaves>(local, wave_tot[0], &tot);
      if (above < want && want <= above + local) {
        // the cut is in this thread's bins: walk them from the highest digit
        uint32_t run = above;
#pragma unroll
        for (int q = kBinsPerThread - 1; q >= 0; --q) {
          if (run < want && want <= run + h[q]) {
            pick_digit = (uint32_t)(bin0 + q);
            pick_above = run;
            pick_count = h[q];
          }
          run += h[q];
        }
      }
#pragma unroll
      for (int q = 0; q < kBinsPerThread / 4; ++q) hist4[bin0 / 4 + q] = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
      prefix |= pick_digit << lo;
      want -= pick_above;
      tshift = (uint32_t)lo;
      if (pick_count == want) break;  // the whole bin is taken
      hi = lo - 1;
    }
  }
  const uint32_t T = prefix >> tshift;

  // taken: forced, competing keys above T, and of the keys equal to T the
  // `want` with the lowest ids
  uint32_t sure = forced, eq = 0;
  if (want > 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t kt = key[j] >> tshift;
      if ((cand >> j) & 1u) {
        if (kt > T) sure |= 1u << j;
        else if (kt == T) eq |= 1u << j;
      }
    }
  }
  uint32_t total;
  const uint32_t packed = ((uint32_t)__builtin_popcount(sure) << 16) | (uint32_t)__builtin_popcount(eq);
  const uint32_t ex = block_scan<kTopkWaves>(packed, wave_tot[1], &total);
  // equal keys taken by lower threads, and how many are left for this one
  // (no conditional subtraction here: hipcc's optimizer turned the form
  // `want > x ? min(n, want - x) : 0` into one that dropped the min below)
  const uint32_t eq_taken_before = min(ex & 0xFFFFu, want);
  uint32_t take_eq = min((uint32_t)__builtin_popcount(eq), want - eq_taken_before);
  uint32_t taken = sure;
  for (uint32_t e = eq; take_eq > 0; --take_eq) {  // the lowest take_eq equal keys
    const uint32_t low = e & (0u - e);
    taken |= low;
    e ^= low;
  }
  uint32_t pos = (ex >> 16) + eq_taken_before;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((taken >> j) & 1u) {
      if (pos < (uint32_t)K) {
        ids[pos] = b0 + j;
        sc[pos] = sv[j];
      }
      ++pos;
    }
  }
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The same selection with one wave a row, for rows of at most 64 S blocks:
// lane l holds blocks l, l + 64, ... (slot j: block 64 j + l).  The
// want-th largest competing key T is found by a radix select over 8-bit
// digits with a 256-bin histogram in LDS per wave (or, with
// IDX_TOPK_RADIX 0, bit by bit from the top: a candidate threshold c >= 1 is
// kept when at least `want` competing keys reach it; blocks that do not
// compete hold key 0, below every c).  Keys equal to T are taken lowest id
// first, and the output positions (ascending ids) come from ballot masks.
// (A resident grid of these waves walking the rows, each loading its next
// row's scores during the current selection, measured 20 % slower: the loop
// state spilled scalar registers and cost occupancy.)

// The selection of row o; hw: the wave's histogram.
template <int S>
__device__ __forceinline__ void ballot_row(const StepArgs& a, int64_t o, int rows, int K, int MB, int lane,
                                           uint32_t* hw) {
  const int r = (int)(o / rows), i = (int)(o - (int64_t)r * rows);
  const float* bs = a.block_scores + o * MB;
  const int slot = a.req_slot[r];
  const int len_raw = a.row_len[r * a.P + i / a.H];
#if IDX_TOPK_BALLOT_SCHED
  __builtin_amdgcn_sched_barrier(0);
#endif
  // the row's scores are loaded up to max_blocks without waiting for the
  // slot and the length (every column of the row is written), so the two
  // loads overlap instead of following each other
  float sv[S];
#if IDX_TOPK_BALLOT_BUFLOAD
  // through a descriptor of the row (max_blocks floats): past it a load
  // returns 0, and those blocks are past nb too, so nothing reads them
  const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(bs), (short)0, 4 * MB,
                                                                        0x00020000);
#pragma unroll
  for (int j = 0; j < S; ++j)
    sv[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rrow, 4 * (64 * j + lane), 0, 0));
#else
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int b = 64 * j + lane;
    sv[j] = b < MB ? bs[b] : -INFINITY;
  }
#endif
  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  const int nb = pad ? 0 : blocks_of(clamp_len(len_raw, MB));
  int32_t* ids = a.topk_ids + o * K;
  float* sc = a.topk_scores + o * K;
  if (nb <= K) {
    for (int t = lane; t < K; t += 64) {
      ids[t] = t < nb ? t : -1;
      sc[t] = t < nb ? bs[t] : -INFINITY;
    }
    return;
  }

  const int init = a.init_blocks, local_from = nb - a.local_blocks;
  uint32_t key[S], ckey[S];  // ckey: the key where the block competes, else 0
  uint32_t cand = 0, forced = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int b = 64 * j + lane;
    const bool in = b < nb;
    key[j] = order_key(sv[j]);
    const bool f = in && (b < init || b >= local_from);
    const bool c = in && !f;
    forced |= (uint32_t)f << j;
    cand |= (uint32_t)c << j;
    ckey[j] = c ? key[j] : 0u;
    if (c) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  // nb > K >= init + local: the two forced ranges exist whole and do not overlap
  const uint32_t want = (uint32_t)(K - init - a.local_blocks);

  // T: the want-th largest competing key.  Every threshold tried is >= 1;
  // T stays 0 only when fewer than `want` competing keys are above 0 (NaN
  // scores have key 0).  The bits above the highest one in which the
  // competing keys differ are theirs in common.
  uint32_t T = 0u;
  if (want > 0) {
    kmin = wave_reduce<0>(kmin);
    kmax = wave_reduce<1>(kmax);
    int hi = 31;
    if (kmin != kmax) {
      hi = 31 - __builtin_clz(kmin ^ kmax);
      T = (hi == 31) ? 0u : (kmin >> (hi + 1)) << (hi + 1);
    } else {
      T = kmin;
      hi = -1;
    }
#if IDX_TOPK_RADIX
    // Radix select, 8 bits a pass from bit hi down: count the competing
    // keys that share T's bits above the digit into a 256-bin histogram in
    // LDS, take the highest digit at which the count from the top reaches
    // `need`, and keep the keys above it.  Stop when that digit's bin holds
    // exactly the keys still needed (T = its lower bound selects them) or
    // the last bit is fixed (T is the key itself).  Lane l holds bins
    // 255 - 4 l - 3 .. 255 - 4 l, so an inclusive scan over the lanes
    // counts from the top.
    uint32_t need = want;
    while (hi >= 0) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      reinterpret_cast<u32x4*>(hw)[lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const bool same = (hi == 31) || (((ckey[j] ^ T) >> (hi + 1)) == 0u);
        if (((cand >> j) & 1u) && same) atomicAdd(&hw[(ckey[j] >> lo) & dmask], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const u32x4 c = reinterpret_cast<const u32x4*>(hw)[63 - lane];  // bins 252 - 4 l .. 255 - 4 l
      const uint32_t sum = c.x + c.y + c.z + c.w;
      const uint32_t incl = wave_inclusive_sum(sum);
      const uint32_t a3 = incl - sum + c.w, a2 = a3 + c.z, a1 = a2 + c.y;  // counts from the top
      const bool here = incl >= need && incl - sum < need;                  // the digit is in this lane
      const uint64_t hm = __builtin_amdgcn_ballot_w64(here);
      const int src = (int)__builtin_ctzll(hm);
      // in the found lane: the digit, the keys above it and in its bin
      const uint32_t sel = a3 >= need ? 3u : a2 >= need ? 2u : a1 >= need ? 1u : 0u;
      const uint32_t above = sel == 3u ? incl - sum : sel == 2u ? a3 : sel == 1u ? a2 : a1;
      const uint32_t inbin = sel == 3u ? c.w : sel == 2u ? c.z : sel == 1u ? c.y : c.x;
      const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)(252u - 4u * (uint32_t)lane + sel), src);
      const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
      const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)inbin, src);
      T |= d << lo;
      need -= ab;
      if (ib == need || lo == 0) break;
      hi = lo - 1;
    }
#else
    // unrolled: no loop control among the counting (bits above hi skip).
    // Once exactly `want` keys reach c they are the ones to take, and T = c
    // (a key or not) selects them: keys above T, then all keys equal to it;
    // the lower bits are not needed.  The count runs on the vector unit (per
    // lane, then a DPP sum across the wave): the scalar unit is one a CU,
    // shared by its four SIMDs, and a ballot with a scalar popcount per slot
    // made it the bottleneck.
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      if (bit > hi) continue;
      const uint32_t c = T | (1u << bit);
#if IDX_TOPK_VALU_COUNT
      uint32_t cl = 0;
#pragma unroll
      for (int j = 0; j < S; ++j) cl += (ckey[j] >= c) ? 1u : 0u;
      const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(cl), 63);
#else
      uint32_t n = 0;
#pragma unroll
      for (int j = 0; j < S; ++j) n += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(ckey[j] >= c));
#endif
      if (n >= want) T = c;
      if (n == want) break;
    }
#endif
  }

  // taken: forced, competing keys above T, and of those equal to T the first
  // `rem` in id order (all of them after an early stop); written at their
  // rank in id order
  uint32_t above = 0;
  if (want > 0) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      above += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(((cand >> j) & 1u) && key[j] > T));
  }
  const uint32_t rem = want - above;  // keys equal to T to take
  uint32_t eq_before = 0, sel_before = 0;
  const __amdgpu_buffer_rsrc_t rid = __builtin_amdgcn_make_buffer_rsrc(ids, (short)0, 4 * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(sc, (short)0, 4 * K, 0x00020000);
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool c = (cand >> j) & 1u;
    const bool eq = want > 0 && c && key[j] == T;
    const uint64_t em = __builtin_amdgcn_ballot_w64(eq);
    const bool take =
        ((forced >> j) & 1u) || (want > 0 && c && key[j] > T) || (eq && eq_before + lanes_below(em) < rem);
    const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
    const uint32_t pos = sel_before + lanes_below(tm);
    // exactly K are taken (init + local forced, want competing); a lane with nothing to write
    // stores past the row's descriptor, which drops it (no branch)
    const uint32_t off = (take && pos < (uint32_t)K) ? 4u * pos : 4u * (uint32_t)K;
    __builtin_amdgcn_raw_buffer_store_b32(64 * j + lane, rid, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv[j]), rsc, off, 0, 0);
    eq_before += (uint32_t)__builtin_popcountll(em);
    sel_before += (uint32_t)__builtin_popcountll(tm);
  }
}

template <int S>
__global__ __launch_bounds__(kBallotThreads) void topk_ballot_kernel(const StepArgs a) {
  __shared__ alignas(16) uint32_t ballot_hist[kBallotWaves][256];  // one histogram a wave
  auto hw_of = [&](int w) { return ballot_hist[w]; };
  const int lane = threadIdx.x & 63;
  const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = a.P * a.H;
  const int K = a.topk, MB = a.max_blocks;
  const int64_t o = (int64_t)blockIdx.x * kBallotWaves + wave;
  if (o >= (int64_t)a.n_req * rows) return;
  ballot_row<S>(a, o, rows, K, MB, lane, hw_of(wave));
}

// topk_ballot_kernel for the row's slot count S = ceil(max_blocks / 64), 1..16.
template <int S>
void launch_ballot(const StepArgs& a, int64_t rows, hipStream_t stream) {
  if constexpr (S > 16) {
    (void)a, (void)rows, (void)stream;
  } else if (a.max_blocks > 64 * S) {
    launch_ballot<S + 1>(a, rows, stream);
  } else {
    hipLaunchKernelGGL(topk_ballot_kernel<S>, dim3((unsigned)((rows + kBallotWaves - 1) / kBallotWaves)),
                       dim3(kBallotThreads), 0, stream, a);
  }
}

hipError_t launch_topk(const StepArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_req * a.P * a.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  static_assert(IDX_MAX_BLOCKS <= 16 * kTopkThreads, "16 blocks per thread cover the limit");
  // one wave a row for many rows of <= 1,024 blocks, and for rows of one
  // 64-block slot at any count; otherwise a workgroup of eight waves a row
  // (it measured faster for a few hundred rows of 1,024 blocks, slower for
  // rows of 12)
  if (a.max_blocks <= 16 * 64 && (grid >= IDX_TOPK_BALLOT_ROWS || a.max_blocks <= 64))
    launch_ballot<1>(a, grid, stream);
  else if (a.max_blocks <= 4 * kTopkThreads && grid <= IDX_TOPK_WIDE_ROWS)
    hipLaunchKernelGGL((topk_kernel<4, kTopkThreads>), dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, a);
  else if (a.max_blocks <= 8 * kTopkThreadsNarrow)
    hipLaunchKernelGGL((topk_kernel<8, kTopkThreadsNarrow>), dim3((unsigned)grid), dim3(kTopkThreadsNarrow), 0, stream,
                       a);
  else if (a.max_blocks <= 8 * kTopkThreads)
    hipLaunchKernelGGL((topk_kernel<8, kTopkThreads>), dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_kernel<16, kTopkThreads>), dim3((unsigned)grid), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace idx
