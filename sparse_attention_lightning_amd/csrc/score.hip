// score.hip -- packed block scoring for gfx950 (MI355X).
//
// All of a request's rows (packed_queries x gqa <= 16) form one 16-row MFMA
// tile, so each K page is read from HBM once for every row and head (sglang
// PR 45451, Modifications; sglang PR 42614, Modifications item 1).  The K read
// extent is the group's longest row; masks use each row's own length.  A
// request whose slot lies outside the request table is a graph pad: it reads
// no K.
//
// Work split.  The grid is persistent (as many workgroups as fit on the chip
// at once).  Every workgroup first computes, for all requests, the number of
// blocks the group reads and their prefix sums (in LDS); the N pages of the
// whole step, in (request, block) order, are then cut into equal contiguous
// slices, one per wave.  A wave walks its slice as tasks of at most 64 pages
// of one request, so it pays one start-up per task instead of one per few
// pages, and all waves finish together.
//
// Within a task, lane j holds the page id of the task's page j, and the wave
// streams the task as 64-token halves through a ring of register buffers,
// keeping RING - 1 halves in flight while the matrix cores work on one.
// Loads go through per-page buffer descriptors: a page that must not be read
// (out of range, or past the task) gets an empty descriptor and reads zeros
// without touching memory, so the loads need no branches and the hardware
// wait counters can keep the prefetches in flight.  Each half is four 16-token
// tiles; per tile and per 32-element k-step one MFMA 16x16x32 computes 16 rows
// x 16 tokens.  Lane l: n = l % 16 is the MFMA column (token) and the A-operand
// row, g = l / 16 its k-group; the fp32 result holds rows 4g..4g+3 of token n.
// The k positions a lane feeds are chosen per format so that each lane's loads
// are 16-byte pieces of its own token's row, and Q is loaded with the same
// d -> k assignment:
//   bf16  row 256 B: step s takes d = 32 s + 8 g .. +8       (4 loads / tile)
//   fp8   row 128 B: bytes [16g, +16) and [64 + 16g, +16);  (2 loads / tile)
//         step s: d = 16 g + 8 s (s < 2), 64 + 16 g + 8 (s - 2)
//   nvfp4 row 64 B:  bytes [16g, +16) = d 32 g .. 32 g + 32; (1 load / tile)
//         step s: d = 32 g + 8 s, inside scale group 2 g + s / 2
// fp8 bytes widen exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1).
// NVFP4: v_cvt_scalef32_pk_f16_fp4 applies the exponent of the E4M3 scale and
// v_pk_mul_f16 its mantissa factor; e2m1 x E4M3 products are exact in f16
// (ATOM PR 2745, Validation).  That path multiplies in f16, so the request's
// bf16 queries are converted to f16 under a power-of-two scale 2^sigma that
// puts the tile's largest magnitude in [2^14, 2^15); the fp32 block max is
// scaled back by 2^-sigma, which is exact.
#include "device.h"

namespace idx {

// Tuning knobs (compile-time; none of them changes what is computed).
#ifndef IDX_SCORE_RING
#define IDX_SCORE_RING 0         // half-page buffers per wave, even (0: per-format default)
#endif
#ifndef IDX_SCORE_NT
#define IDX_SCORE_NT 0           // 1: non-temporal (streaming) K loads
#endif
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTaskPages = 64;   // one page id per lane

template <int FMT>
struct Fmt;

template <>
struct Fmt<IDX_K_BF16> {
  // half pages in flight per wave (registers bound it: a bf16 half is 16 KB a wave)
  static constexpr int kRing = IDX_SCORE_RING ? IDX_SCORE_RING : 2;
  static constexpr int kRowBytes = 256;
  static constexpr int kLoads = 4;  // 16-byte loads per lane per tile
  typedef bf16x8 Op;
  __device__ static int d0(int s, int g) { return 32 * s + 8 * g; }
  __device__ static int off(int i, int g) { return 64 * i + 16 * g; }
};

template <>
struct Fmt<IDX_K_FP8_E4M3> {
  // half pages in flight per wave (registers bound it: a bf16 half is 16 KB a wave)
  static constexpr int kRing = IDX_SCORE_RING ? IDX_SCORE_RING : 4;
  static constexpr int kRowBytes = 128;
  static constexpr int kLoads = 2;
  typedef bf16x8 Op;
  __device__ static int d0(int s, int g) { return (s < 2) ? 16 * g + 8 * s : 64 + 16 * g + 8 * (s - 2); }
  __device__ static int off(int i, int g) { return 64 * i + 16 * g; }
};

template <>
struct Fmt<IDX_K_NVFP4> {
  // half pages in flight per wave (registers bound it: a bf16 half is 16 KB a wave)
  static constexpr int kRing = IDX_SCORE_RING ? IDX_SCORE_RING : 4;
  static constexpr int kRowBytes = 64;
  static constexpr int kLoads = 1;
  typedef f16x8 Op;
  __device__ static int d0(int s, int g) { return 32 * g + 8 * s; }
  __device__ static int off(int, int g) { return 16 * g; }
};

// Registers holding one lane's share of a 64-token half page.
template <int FMT>
struct Half {
  u32x4 v[4][Fmt<FMT>::kLoads];
  uint32_t sc[4];  // NVFP4: this lane's two scale bytes of each tile
};

// E4M3 byte (non-negative scales; the sign bit is honoured) to float.
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  float v = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120) << 23) | (m << 20));
  return (b & 0x80) ? -v : v;
}

// Buffer descriptor of one page.  Word 3 is the raw 32-bit data format of
// gfx9 MUBUF descriptors.  A page the kernel must not read gets size 0: every
// load through it is out of range, returns zeros and touches no memory.  Its
// base still points at page 0 of the pool, so even a load that ignored the
// size would stay inside the pool.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* pool, int64_t page,
                                                           bool ok, int bytes) {
  const uint8_t* base = ok ? pool + page * bytes : pool;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, ok ? bytes : 0,
                                           0x00020000);
}

// Load one lane's share of half page `half`: straight-line loads only, so
// the wait counters can keep later units in flight while this one is used.
template <int FMT>
__device__ __forceinline__ void load_half(Half<FMT>& h, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rs, int half, int n, int g) {
  const int tok0 = half * 64 + n;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = (tok0 + 16 * t) * Fmt<FMT>::kRowBytes;
#pragma unroll
    for (int i = 0; i < Fmt<FMT>::kLoads; ++i)
      h.v[t][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, row + Fmt<FMT>::off(i, g), 0,
                                                       IDX_SCORE_NT ? 2 : 0));
    if constexpr (FMT == IDX_K_NVFP4)
      h.sc[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, (tok0 + 16 * t) * 8 + 2 * g, 0, 0);
  }
}

// B operand of k-step s for tile t.
template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Op operand(const Half<FMT>& h, int t, int s,
                                                         const float* scale, const f16x2* mant) {
  if constexpr (FMT == IDX_K_BF16) {
    return __builtin_bit_cast(bf16x8, h.v[t][s]);
  } else if constexpr (FMT == IDX_K_FP8_E4M3) {
    const u32x4 w = h.v[t][s >> 1];
    const uint32_t lo = (s & 1) ? w.z : w.x, hi = (s & 1) ? w.w : w.y;
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 o;
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
    o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
    return o;
  } else {
    const u32x4 w4 = h.v[t][0];
    const uint32_t w = (s == 0) ? w4.x : (s == 1) ? w4.y : (s == 2) ? w4.z : w4.w;
    const float sc = scale[s >> 1];
    const f16x2 m = mant[s >> 1];
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0) * m;
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1) * m;
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2) * m;
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3) * m;
    f16x8 o;
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
    o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
    return o;
  }
}

template <int FMT>
__device__ __forceinline__ f32x4 mfma(typename Fmt<FMT>::Op a, typename Fmt<FMT>::Op b, f32x4 c) {
  if constexpr (FMT == IDX_K_NVFP4)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fold one half page into the running per-row maxima of this lane's 4 rows.
template <int FMT>
__device__ __forceinline__ void score_half(const Half<FMT>& h, const typename Fmt<FMT>::Op* qf,
                                           bool full, int pos0, const int* len, float* mx) {
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // NVFP4: per tile the two scale groups this lane touches
  float scale[4][2];
  f16x2 mant[4][2];
  (void)scale;
  (void)mant;
  if constexpr (FMT == IDX_K_NVFP4) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float s = e4m3_to_float((h.sc[t] >> (8 * q)) & 0xFF);
        scale[t][q] = s;  // the conversion applies the exponent of s
        const _Float16 f = (_Float16)__uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
        mant[t][q] = f16x2{f, f};
      }
  }
  // k-step outer, tile inner: four independent accumulation chains
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mfma<FMT>(qf[s], operand<FMT>(h, t, s, scale[t], mant[t]), acc[t]);
  if (full) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], acc[t][j]);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], (pos0 + 16 * t < len[j]) ? acc[t][j] : -INFINITY);
  }
}

// One task: pages [b_s, b_s + cnt) of request r (cnt <= 64), all P*H rows.
// `stage` is this wave's LDS buffer of kTileRows x kTaskPages block scores:
// the task's results are collected there and written out row by row, so
// every row leaves as one contiguous run instead of one 4-byte store per page.
template <int FMT>
__device__ __forceinline__ void score_task(const StepArgs& a, int r, int b_s, int cnt, int lane,
                                           int n, int g, float* stage) {
  typedef typename Fmt<FMT>::Op Op;
  const int P = a.P, H = a.H, rows = P * H, MB = a.max_blocks;
  const int slot = a.req_slot[r];  // a task never belongs to a graph pad
  const int32_t* bt = a.block_table + (int64_t)slot * MB + b_s;
  const int pidv = (lane < cnt) ? bt[lane] : -1;  // lane j: page id of the task's page j

  int lmin = MB * kBlock;
  for (int j = 0; j < P; ++j) lmin = min(lmin, clamp_len(a.row_len[r * P + j], MB));
  int len[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * g + j;
    len[j] = (row < rows) ? clamp_len(a.row_len[r * P + row / H], MB) : 0;
  }
  const int wrow = 4 * g + n;  // lanes n < 4 hold row 4g + n
  const bool writer = n < 4 && wrow < rows;
  const int my_len = (n == 0) ? len[0] : (n == 1) ? len[1] : (n == 2) ? len[2] : len[3];

  // Q fragments: A operand row n, k-group g
  Op qf[4];
  int sigma = 0;
  const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)r * rows + n) * kHeadDim;
  if constexpr (FMT == IDX_K_NVFP4) {
    bf16x8 qb[4];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qb[s] = (n < rows) ? *reinterpret_cast<const bf16x8*>(qrow + Fmt<FMT>::d0(s, g)) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qb[s][e]));
    }
    amax = row16_max(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);  // amax < 2^ex
      sigma = 15 - ex;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (_Float16)ldexpf((float)qb[s][e], sigma);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = (n < rows) ? *reinterpret_cast<const Op*>(qrow + Fmt<FMT>::d0(s, g)) : Op{};
  }

  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* ks = a.k_scale;
  constexpr int kPageBytes = kBlock * Fmt<FMT>::kRowBytes;
  constexpr int kRing = Fmt<FMT>::kRing;
  static_assert(kRing == 2 || kRing == 4, "an even ring of 2 or 4 half pages");
  const int n_units = 2 * cnt;  // unit u: half u % 2 of task page u / 2

  // issue the loads of unit ua (any ua: past the task it reads zeros)
  auto issue = [&](Half<FMT>& h, int ua) {
    const int j = ua >> 1;
    const int pid = __builtin_amdgcn_readlane(pidv, min(j, kTaskPages - 1));
    const bool ok = j < cnt && pid >= 0 && pid < a.n_pages;
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(kp, pid, ok, kPageBytes);
    const __amdgpu_buffer_rsrc_t rs = (FMT == IDX_K_NVFP4) ? page_rsrc(ks, pid, ok, kBlock * 8) : rk;
    load_half<FMT>(h, rk, rs, ua & 1, n, g);
  };

  Half<FMT> ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) issue(ring[u], u);
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int u0 = 0; u0 < n_units; u0 += kRing) {
    // kRing units per trip (even), so ring slots and halves are static
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int u = u0 + k;
      issue(ring[(k + kRing - 1) % kRing], u + kRing - 1);
      const int j = u >> 1;
      const int b = b_s + j;
      if ((k & 1) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) mx[e] = -INFINITY;
      }
      const bool full = (b + 1) * kBlock <= lmin;
      score_half<FMT>(ring[k], qf, full, b * kBlock + 64 * (k & 1) + n, len, mx);
      if (k & 1) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = row16_max(mx[e]);
        float o = (n == 0) ? v[0] : (n == 1) ? v[1] : (n == 2) ? v[2] : v[3];
        if constexpr (FMT == IDX_K_NVFP4) o = ldexpf(o, -sigma);
        const int pid = __builtin_amdgcn_readlane(pidv, min(j, kTaskPages - 1));
        if (!(pid >= 0 && pid < a.n_pages)) o = (b * kBlock < my_len) ? __builtin_nanf("") : -INFINITY;
        if (writer && j < cnt) stage[wrow * kTaskPages + j] = o;
      }
    }
  }
  // write the task's scores: row i, blocks [b_s, b_s + cnt), one lane per block
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  float* out = a.block_scores + (int64_t)r * rows * MB + b_s;
  for (int i = 0; i < rows; ++i)
    if (lane < cnt) out[(int64_t)i * MB + lane] = stage[i * kTaskPages + lane];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void score_kernel(const StepArgs a) {
  extern __shared__ uint32_t pre[];  // n_req + 1 prefix sums of per-request block counts
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ float stage[kWaves][kTileRows * kTaskPages];
  // Values that are uniform across a wave are passed through readfirstlane so
  // the compiler keeps them (and the buffer descriptors built from them) in
  // scalar registers.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int P = a.P, rows = P * a.H, MB = a.max_blocks, R = a.n_req;

  // 1. blocks each request's group reads (0 for graph pads), prefix sums
  uint32_t carry = 0;
  for (int base = 0; base < R; base += kThreads) {
    const int r = base + tid;
    uint32_t nbg = 0;
    if (r < R) {
      const int slot = a.req_slot[r];
      if (slot >= 0 && slot < a.n_slot_rows) {
        int lmax = 0;
        for (int j = 0; j < P; ++j) lmax = max(lmax, clamp_len(a.row_len[r * P + j], MB));
        nbg = (uint32_t)blocks_of(lmax);
      }
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kThreads>(nbg, wave_tot, &tot);
    if (r < R) pre[r] = carry + ex;
    carry += tot;
  }
  if (tid == 0) pre[R] = carry;
  __syncthreads();
  const uint32_t N = __builtin_amdgcn_readfirstlane(carry);

  // 2. -inf past each group's extent, and everywhere for graph pads
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int nbg = (int)(__builtin_amdgcn_readfirstlane(pre[r + 1]) -
                          __builtin_amdgcn_readfirstlane(pre[r]));
    const int width = MB - nbg;
    float* base = a.block_scores + (int64_t)r * rows * MB + nbg;
    for (int e = tid; e < rows * width; e += kThreads) base[(int64_t)(e / width) * MB + e % width] = -INFINITY;
  }

  // 3. this wave's equal share of the N pages, as tasks of one request each
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t wid = (int64_t)blockIdx.x * kWaves + wave;
  int64_t pos = wid * N / nw;
  const int64_t end = (wid + 1) * N / nw;
  if (a.n_pages == 0) {
    // nothing can be read: every visible block is NaN
    for (; pos < end; ++pos) {
      int lo = 0, hi = R;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)__builtin_amdgcn_readfirstlane(pre[mid]) <= pos) lo = mid; else hi = mid;
      }
      const int b = (int)(pos - __builtin_amdgcn_readfirstlane(pre[lo]));
      const int wrow = 4 * g + n;
      if (n < 4 && wrow < rows) {
        const int L = clamp_len(a.row_len[lo * P + wrow / a.H], MB);
        a.block_scores[((int64_t)lo * rows + wrow) * MB + b] = (b * kBlock < L) ? __builtin_nanf("") : -INFINITY;
      }
    }
    return;
  }
  while (pos < end) {
    int lo = 0, hi = R;  // the request holding page pos: pre[lo] <= pos < pre[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)__builtin_amdgcn_readfirstlane(pre[mid]) <= pos) lo = mid; else hi = mid;
    }
    const int64_t first = __builtin_amdgcn_readfirstlane(pre[lo]);
    const int b_s = (int)(pos - first);
    const int nbg = (int)(__builtin_amdgcn_readfirstlane(pre[lo + 1]) - first);
    const int cnt = (int)min<int64_t>(min<int64_t>(end - pos, nbg - b_s), kTaskPages);
    score_task<FMT>(a, lo, b_s, cnt, lane, n, g, stage[wave]);
    pos += cnt;
  }
}

namespace {
// workgroups that fit on the device at once for this kernel (cached per device)
template <int FMT>
int resident_workgroups(size_t smem) {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(score_kernel<FMT>),
                                                   kThreads, smem) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev] = cus * per_cu;
  return cache[dev];
}
}  // namespace

hipError_t launch_score(const StepArgs& a, hipStream_t stream) {
  if (a.n_req == 0 || a.max_blocks == 0) return hipSuccess;
  const size_t smem = (size_t)(IDX_MAX_REQ + 1) * sizeof(uint32_t);  // sized for the limit
  switch (a.k_format) {
    case IDX_K_BF16:
      hipLaunchKernelGGL(score_kernel<IDX_K_BF16>, dim3(resident_workgroups<IDX_K_BF16>(smem)),
                         dim3(kThreads), smem, stream, a);
      break;
    case IDX_K_FP8_E4M3:
      hipLaunchKernelGGL(score_kernel<IDX_K_FP8_E4M3>, dim3(resident_workgroups<IDX_K_FP8_E4M3>(smem)),
                         dim3(kThreads), smem, stream, a);
      break;
    default:
      hipLaunchKernelGGL(score_kernel<IDX_K_NVFP4>, dim3(resident_workgroups<IDX_K_NVFP4>(smem)),
                         dim3(kThreads), smem, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace idx
