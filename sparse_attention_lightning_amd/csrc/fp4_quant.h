// fp4_quant.h -- the NVFP4 key quantizer shared by the store kernels and the
// score kernel's fused store of a step's new keys.
//
// ROCm/ATOM PR 2745, Summary ("Store" and the per-key layout): per 16-element
// group, scale = e4m3(amax / 6) and codes rounded half-to-even, saturating at
// 6; two codes a byte, the even element in the low nibble; 64 B payload and
// 8 B scales per key, written at the key's slot.  amax / 6 is an IEEE fp32
// division; its E4M3 rounding (nearest, ties to even, clamped at 448) is done
// on the bits.  Codes come from exact comparisons of |x| with the e2m1
// midpoints times the scale (each product is exact in fp32), which is the
// half-to-even rounding of x / scale without a division.  A code keeps the
// sign bit of x; a zero scale gives magnitude 0.
#pragma once

#include "device.h"

namespace idx {

__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float t) {
  if (!(t < 448.0f)) return 0x7Eu;  // clamp (NaN too: unspecified)
  if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);  // subnormal step 2^-9
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round to 3 mantissa bits, ties to even
  const uint32_t e = (u >> 23) - 127u + 7u;
  return (e << 3) | ((u >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// One 16-element group: its E4M3 scale byte and its 16 codes, two a byte
// (the even element in the low nibble) in packed[0..1].
__device__ __forceinline__ uint32_t quantize16(u32x4 w0, u32x4 w1, uint32_t* packed) {
  const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float x[16];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = __uint_as_float(wd[j] << 16);
    x[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
    amax = fmaxf(amax, fmaxf(fabsf(x[2 * j]), fabsf(x[2 * j + 1])));
  }
  const uint32_t sb = e4m3_rne_satfinite(amax / 6.0f);
  const float s = e4m3_value(sb);
  // midpoints of the e2m1 grid 0 .5 1 1.5 2 3 4 6, times s (exact); a zero
  // scale makes them infinite, so every code has magnitude 0
  const float sz = s > 0.0f ? s : __builtin_inff();
  float m0 = 0.25f * sz, m1 = 0.75f * sz, m2 = 1.25f * sz, m3 = 1.75f * sz;
  float m4 = 2.5f * sz, m5 = 3.5f * sz, m6 = 5.0f * sz;
  // keep the seven products in registers: otherwise the compiler selects the
  // constant per value and multiplies it again
  asm volatile("" : "+v"(m0), "+v"(m1), "+v"(m2), "+v"(m3), "+v"(m4), "+v"(m5), "+v"(m6));
  packed[0] = packed[1] = 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float a = fabsf(x[j]);
    // ties: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    const bool b2 = a >= m3;
    const bool b1 = a >= (b2 ? m5 : m1);
    const float t3 = b2 ? (b1 ? m6 : m4) : (b1 ? m2 : m0);
    const uint32_t mag = (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + (a > t3 ? 1u : 0u);
    const uint32_t code = mag | ((__float_as_uint(x[j]) >> 28) & 8u);
    packed[j >> 3] |= code << (4 * (j & 7));
  }
  return sb;
}

// Quantize one group (this lane's) of a key and store it; the key's eight
// lanes call this together.
template <bool NT = false>
__device__ __forceinline__ void quantize_group(u32x4 w0, u32x4 w1, int64_t slot, int grp, uint8_t* payload,
                                               uint8_t* scales) {
  uint32_t packed[2];
  const uint32_t sb = quantize16(w0, w1, packed);
  u32x2* pdst = reinterpret_cast<u32x2*>(payload + slot * 64 + 8 * grp);
  // the key's 8 scale bytes as one 8-byte store from its first lane: each
  // quad of lanes ORs its bytes into a word, lane 4 hands its word to lane 0
  uint32_t word = sb << (8 * (grp & 3));
  word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  const uint32_t hi = __shfl_down(word, 4, 8);
  u32x2* sdst = reinterpret_cast<u32x2*>(scales + slot * 8);
  if constexpr (NT) {
    __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, pdst);
    if (grp == 0) __builtin_nontemporal_store(u32x2{word, hi}, sdst);
  } else {
    *pdst = u32x2{packed[0], packed[1]};
    if (grp == 0) *sdst = u32x2{word, hi};
  }
}

}  // namespace idx
