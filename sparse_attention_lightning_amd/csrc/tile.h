// tile.h -- the 16-row query tile against K pages, shared by the gfx950
// scoring kernels (device code only).
//
// A wave works on 64-token halves of a page.  Loads from HBM go through
// per-page buffer descriptors: a page that must not be read (out of range, or
// no page at all) gets an empty descriptor and reads zeros without touching
// memory, so the loads need no branches and the hardware wait counters can
// keep the prefetches in flight.  Each half is
// four 16-token tiles; per tile and per 32-element k-step one MFMA 16x16x32
// computes 16 rows x 16 tokens.  Lane l: n = l % 16 is the MFMA column (token)
// and the A-operand row, g = l / 16 its k-group; the fp32 result holds rows
// 4g..4g+3 of token n.  The k positions a lane feeds are chosen per format so
// that each lane's loads are 16-byte pieces of its own token's row, and Q is
// read with the same d -> k assignment:
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
#pragma once

#include "device.h"

namespace idx {

// Tuning knobs (compile-time; none of them changes what is computed).
#ifndef IDX_SCORE_RING_BF16
#define IDX_SCORE_RING_BF16 2    // half-page register buffers per wave, bf16 K (16 KB a wave each)
#endif
#ifndef IDX_SCORE_RING_FP8
#define IDX_SCORE_RING_FP8 4     // fp8 K (8 KB a wave each)
#endif
#ifndef IDX_SCORE_RING_FP4
#define IDX_SCORE_RING_FP4 4     // NVFP4 K (4.5 KB a wave each, with scales)
#endif
#ifndef IDX_SCORE_NT
#define IDX_SCORE_NT 0           // 1: non-temporal (streaming) K loads
#endif
template <int FMT>
struct Fmt;

template <>
struct Fmt<IDX_K_BF16> {
  static constexpr int kRing = IDX_SCORE_RING_BF16;
  static constexpr int kRowBytes = 256;
  static constexpr int kLoads = 4;  // 16-byte loads per lane per tile
  typedef bf16x8 Op;
  __device__ static int d0(int s, int g) { return 32 * s + 8 * g; }
  __device__ static int off(int i, int g) { return 64 * i + 16 * g; }
};

template <>
struct Fmt<IDX_K_FP8_E4M3> {
  static constexpr int kRing = IDX_SCORE_RING_FP8;
  static constexpr int kRowBytes = 128;
  static constexpr int kLoads = 2;
  typedef bf16x8 Op;
  __device__ static int d0(int s, int g) { return (s < 2) ? 16 * g + 8 * s : 64 + 16 * g + 8 * (s - 2); }
  __device__ static int off(int i, int g) { return 64 * i + 16 * g; }
};

template <>
struct Fmt<IDX_K_NVFP4> {
  static constexpr int kRing = IDX_SCORE_RING_FP4;
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

// NVFP4: the two scale groups of each tile this lane touches, as the f32
// scale (the fp4 conversion applies its exponent) and the f16 factor 1.m of
// its mantissa (at most 3 bits, exact in f16).
template <int FMT>
struct Scales {
  float scale[4][2];
  f16x2 mant[4][2];
};

template <int FMT>
__device__ __forceinline__ Scales<FMT> half_scales(const Half<FMT>& h) {
  Scales<FMT> sc;
  if constexpr (FMT == IDX_K_NVFP4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // the two scale bytes through the hardware E4M3 conversion (unit scale)
      sc.scale[t][0] = __builtin_amdgcn_cvt_scalef32_f32_fp8(h.sc[t], 1.0f, 0);
      sc.scale[t][1] = __builtin_amdgcn_cvt_scalef32_f32_fp8(h.sc[t], 1.0f, 1);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const _Float16 f =
            (_Float16)__uint_as_float((__float_as_uint(sc.scale[t][q]) & 0x007FFFFFu) | 0x3F800000u);
        sc.mant[t][q] = f16x2{f, f};
      }
    }
  }
  return sc;
}

// NT 16-row query tiles against one half page: acc[u][t] holds tile u's rows
// 4g..4g+3 x token n of 16-token tile t.  Each K operand is decoded once and
// feeds the NT tiles' MFMAs.
template <int FMT, int NT>
__device__ __forceinline__ void half_dot(const Half<FMT>& h, const typename Fmt<FMT>::Op (*qf)[4],
                                         f32x4 (*acc)[4]) {
  const Scales<FMT> sc = half_scales<FMT>(h);
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // k-step outer, tile inner: independent accumulation chains
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const typename Fmt<FMT>::Op op = operand<FMT>(h, t, s, sc.scale[t], sc.mant[t]);
#pragma unroll
      for (int u = 0; u < NT; ++u) acc[u][t] = mfma<FMT>(qf[u][s], op, acc[u][t]);
    }
}

// Fold one half page's dot products into the running state of this lane's 4
// rows.
// IDX_SCORE_MAX: st0 = the running max of q.k.  IDX_SCORE_LSE: st0 = the
// running max m of v = c2 * q.k and st1 = the sum of 2^(v - m) (c2 carries
// sm_scale, log2 e and, for NVFP4, the query tile's 2^-sigma).
template <int MODE>
__device__ __forceinline__ void fold(const f32x4* acc, bool full, int pos0, const int* len, float* st0,
                                     float* st1, float c2) {
  if constexpr (MODE == IDX_SCORE_MAX) {
    (void)st1;
    (void)c2;
    if (full) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) st0[j] = fmaxf(st0[j], acc[t][j]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) st0[j] = fmaxf(st0[j], (pos0 + 16 * t < len[j]) ? acc[t][j] : -INFINITY);
    }
  } else if (full) {
    // every token visible: the new max is finite (c2 > 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float am = fmaxf(fmaxf(acc[0][j], acc[1][j]), fmaxf(acc[2][j], acc[3][j]));
      const float mnew = fmaxf(st0[j], am * c2);
      float sum = st1[j] * __builtin_amdgcn_exp2f(st0[j] - mnew);  // 0 while st0 is -inf
#pragma unroll
      for (int t = 0; t < 4; ++t) sum += __builtin_amdgcn_exp2f(fmaf(acc[t][j], c2, -mnew));
      st1[j] = sum;
      st0[j] = mnew;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (pos0 + 16 * t < len[j]) ? acc[t][j] * c2 : -INFINITY;
      const float mnew = fmaxf(st0[j], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
      const float base = (mnew == -INFINITY) ? 0.f : mnew;  // nothing visible yet: every term is 0
      float sum = st1[j] * __builtin_amdgcn_exp2f(st0[j] - base);
#pragma unroll
      for (int t = 0; t < 4; ++t) sum += __builtin_amdgcn_exp2f(v[t] - base);
      st1[j] = sum;
      st0[j] = mnew;
    }
  }
}

// One 16-row tile against one half page: dot products and fold.
template <int FMT, int MODE>
__device__ __forceinline__ void score_half(const Half<FMT>& h, const typename Fmt<FMT>::Op* qf,
                                           bool full, int pos0, const int* len, float* st0, float* st1,
                                           float c2) {
  f32x4 acc[1][4];
  half_dot<FMT, 1>(h, reinterpret_cast<const typename Fmt<FMT>::Op(*)[4]>(qf), acc);
  fold<MODE>(acc[0], full, pos0, len, st0, st1, c2);
}


}  // namespace idx
