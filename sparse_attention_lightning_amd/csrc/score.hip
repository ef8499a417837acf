// score.hip -- packed block scoring for gfx950 (MI355X).
//
// One workgroup scores one request over a chunk of 32 blocks.  All of the
// request's rows (packed_queries x gqa <= 16) form one 16-row MFMA tile, so
// each K page is read from HBM once for every row and head (sglang PR 45451,
// Modifications; sglang PR 42614, Modifications item 1).  The K read extent is
// the group's longest row; masks use each row's own length.  A request whose
// slot lies outside the request table is a graph pad: it reads no K.
//
// Wave layout.  Four waves per workgroup, each owns 8 consecutive blocks and
// streams them as 64-token halves, prefetching the next half into registers
// while the matrix cores work on the current one.  Each half is four 16-token
// tiles; per tile and per 32-element k-step one MFMA 16x16x32 computes the
// 16 rows x 16 tokens.  Lane l: n = l % 16 is the MFMA column (token) and the
// A-operand row, g = l / 16 its k-group; the fp32 result holds rows 4g..4g+3
// of token n.  The k positions a lane feeds are chosen per format so that
// each lane's loads are 16-byte pieces of its own token's row, and Q is
// loaded with the same d -> k assignment:
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
#ifndef IDX_SCORE_WAVES
#define IDX_SCORE_WAVES 4        // waves per workgroup
#endif
#ifndef IDX_SCORE_PAGES_PER_WAVE
#define IDX_SCORE_PAGES_PER_WAVE 8
#endif
#ifndef IDX_SCORE_RING
#define IDX_SCORE_RING 0         // half-page buffers per wave (0: per-format default)
#endif
#ifndef IDX_SCORE_NT
#define IDX_SCORE_NT 0           // 1: non-temporal K loads
#endif
constexpr int kWaves = IDX_SCORE_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kPagesPerWave = IDX_SCORE_PAGES_PER_WAVE;
constexpr int kChunkPages = kWaves * kPagesPerWave;


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
  static constexpr int kRing = IDX_SCORE_RING ? IDX_SCORE_RING : 3;
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

template <int FMT>
__device__ __forceinline__ void load_half(Half<FMT>& h, const uint8_t* __restrict__ k,
                                          const uint8_t* __restrict__ ks, int64_t page, int half,
                                          int n, int g) {
  const int64_t tok0 = page * kBlock + half * 64 + n;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint8_t* row = k + (tok0 + 16 * t) * Fmt<FMT>::kRowBytes;
#pragma unroll
    for (int i = 0; i < Fmt<FMT>::kLoads; ++i) {
      const u32x4* src = reinterpret_cast<const u32x4*>(row + Fmt<FMT>::off(i, g));
      h.v[t][i] = IDX_SCORE_NT ? __builtin_nontemporal_load(src) : *src;
    }
    if constexpr (FMT == IDX_K_NVFP4)
      h.sc[t] = *reinterpret_cast<const uint16_t*>(ks + (tok0 + 16 * t) * 8 + 2 * g);
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

template <int FMT>
__global__ __launch_bounds__(kThreads) void score_kernel(const StepArgs a) {
  typedef typename Fmt<FMT>::Op Op;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int r = blockIdx.x / a.n_chunks;
  const int chunk = blockIdx.x - r * a.n_chunks;
  const int P = a.P, H = a.H, rows = P * H, MB = a.max_blocks;
  const int b_begin = chunk * kChunkPages + wave * kPagesPerWave;
  const int b_end = min(b_begin + kPagesPerWave, MB);
  if (b_begin >= b_end) return;

  const int slot = a.req_slot[r];
  const bool pad = slot < 0 || slot >= a.n_slot_rows;
  int lmax = 0, lmin = MB * kBlock;
  for (int j = 0; j < P; ++j) {
    const int L = clamp_len(a.row_len[r * P + j], MB);
    lmax = max(lmax, L);
    lmin = min(lmin, L);
  }
  const int nbg = pad ? 0 : blocks_of(lmax);
  int len[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * g + j;
    len[j] = (row < rows && !pad) ? clamp_len(a.row_len[r * P + row / H], MB) : 0;
  }
  const int wrow = 4 * g + n;  // lanes n < 4 write row 4g + n
  const bool writer = n < 4 && wrow < rows;
  float* wptr = a.block_scores + ((int64_t)r * rows + (writer ? wrow : 0)) * MB;
  const int my_len = (n == 0) ? len[0] : (n == 1) ? len[1] : (n == 2) ? len[2] : len[3];

  const int b_load_end = min(b_end, nbg);
  if (b_begin < b_load_end) {
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

    const int32_t* bt = a.block_table + (int64_t)slot * MB;
    const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
    const uint8_t* ks = a.k_scale;
    int64_t pid[kPagesPerWave];
    bool ok[kPagesPerWave];
#pragma unroll
    for (int i = 0; i < kPagesPerWave; ++i) {
      pid[i] = (b_begin + i < b_load_end) ? bt[b_begin + i] : 0;
      ok[i] = pid[i] >= 0 && pid[i] < a.n_pages;
    }

    // Units are half pages: unit u is half u % 2 of the wave's page u / 2.
    // A ring of kRing buffers keeps kRing - 1 units in flight ahead of the
    // one the matrix cores work on.
    const int n_units = 2 * (b_load_end - b_begin);
    constexpr int kRing = Fmt<FMT>::kRing;
    static_assert(kRing >= 2 && kRing <= 4, "ring of 2..4 half pages");
    Half<FMT> ring[kRing];
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u)
      if (u < n_units && ok[u >> 1]) load_half<FMT>(ring[u], kp, ks, pid[u >> 1], u & 1, n, g);
    float mx[4];
    // constant trip count with uniform guards (no break), so the loop unrolls
    // and every ring / page index is static
#pragma unroll
    for (int u = 0; u < 2 * kPagesPerWave; ++u) {
      if (u < n_units) {
        const int ahead = u + kRing - 1;
        if (ahead < 2 * kPagesPerWave && ahead < n_units && ok[ahead >> 1])
          load_half<FMT>(ring[ahead % kRing], kp, ks, pid[ahead >> 1], ahead & 1, n, g);
        const int i = u >> 1;
        const int b = b_begin + i;
        if ((u & 1) == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) mx[j] = -INFINITY;
        }
        const bool full = (b + 1) * kBlock <= lmin;
        score_half<FMT>(ring[u % kRing], qf, full, b * kBlock + 64 * (u & 1) + n, len, mx);
        if (u & 1) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = row16_max(mx[j]);
          float o = (n == 0) ? v[0] : (n == 1) ? v[1] : (n == 2) ? v[2] : v[3];
          if constexpr (FMT == IDX_K_NVFP4) o = ldexpf(o, -sigma);
          if (!ok[i]) o = (b * kBlock < my_len) ? __builtin_nanf("") : -INFINITY;
          if (writer) wptr[b] = o;
        }
      }
    }
  }
  // blocks past the group's longest row (and every block of a graph pad)
  for (int b = max(b_begin, nbg); b < b_end; ++b)
    if (writer) wptr[b] = -INFINITY;
}

hipError_t launch_score(const StepArgs& a0, hipStream_t stream) {
  StepArgs a = a0;
  a.n_chunks = (a.max_blocks + kChunkPages - 1) / kChunkPages;
  const int64_t grid = (int64_t)a.n_req * a.n_chunks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  switch (a.k_format) {
    case IDX_K_BF16:
      hipLaunchKernelGGL(score_kernel<IDX_K_BF16>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    case IDX_K_FP8_E4M3:
      hipLaunchKernelGGL(score_kernel<IDX_K_FP8_E4M3>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(score_kernel<IDX_K_NVFP4>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace idx
