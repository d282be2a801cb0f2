// MXFP8 element and scale encoding on the device.
//
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上", section
// "MXFP8 および NVFP4 量子化の融合による露出メモリオーバーヘッドの削減": GEMM
// outputs are quantized to MXFP8 in the epilogue, with a transposed copy for
// the backward pass.  The format is the one of the OCP Microscaling Formats
// (MX) Specification v1.0:
//   * E4M3 element: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
//     infinities, S.1111.111 = NaN, largest magnitude 448, subnormal quantum
//     2^-9;
//   * E8M0 scale: 2^(code - 127);
//   * a block of 32 values with largest magnitude amax shares the exponent
//     e = floor(log2 amax) - 8 (8 = exponent of E4M3's largest normal),
//     clamped to [-127, 127], and e = -127 for amax = 0; each value is
//     v / 2^e rounded to nearest even E4M3, saturated to +-448.
// MXFP4 (same specification) uses E2M1 elements: sign, 2 exponent bits (bias
// 1), 1 mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, no NaN; the block
// exponent is floor(log2 amax) - 2 (2 = exponent of 6); codes are packed two
// per byte, element 2 i in the low nibble of byte i; a NaN input becomes the
// largest magnitude with its sign.
// Everything below is exact integer / power-of-two arithmetic on float32.
#pragma once

#include <stdint.h>

namespace moe {

// Shared exponent of a block from its largest magnitude (finite, >= 0);
// EMAX is the exponent of the element format's largest normal.
template <int EMAX = 8>
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23) & 0xff;  // 0 for zero and float32 subnormals
  if (ef == 0) return -127;              // floor(log2 amax) <= -127 -> clamped
  const int e = ef - 127 - EMAX;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as a float32 (e in [-127, 125] for any finite float32 amax, so the
// result is a normal float32 and the scaling is exact).
__device__ __forceinline__ float mx_inv_scale(int e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// E4M3 code of a float32 value (already divided by the block scale): round to
// nearest even, saturate at 448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                 // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;         // |v| >= 448: saturate
  if (a < 0x3c800000u) {                             // |v| < 2^-6: subnormal range
    // quantum 2^-9: code = round_even(|v| * 512); 8 is the smallest normal,
    // whose code is also 8
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)q;
  }
  // normal range: keep 3 mantissa bits, round to nearest even at bit 20, then
  // move the float32 exponent bias (127) to E4M3's (7)
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - ((127u - 7u) << 3));
}

// E2M1 code of a float32 value (already divided by the block scale): round
// to nearest even, saturate at 6.  Each comparison adds one step; the ties
// (0.25, 0.75, ...) fall to the neighbour with the even code.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 28) & 0x8u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  if (a != a) return sign | 7u;
  return sign | (uint32_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                           (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
}

// Four E4M3 codes in one word (value q in byte q) with the hardware
// conversion: round to nearest even, subnormal quantum 2^-9, after clamping
// to +-448 (the saturation rule above).  A NaN among the four takes the
// encoder above (the conversion's NaN code is not the one chosen here).  The
// two agree bit for bit on every other float32 input (checked on the device
// over 18M values: all tie patterns and their neighbours from 2^-32 to 2^13,
// subnormals, infinities, the saturation range).
__device__ __forceinline__ uint32_t e4m3_pack4_soft(float a, float b, float c, float d) {
  return e4m3_code(a) | (e4m3_code(b) << 8) | (e4m3_code(c) << 16) | (e4m3_code(d) << 24);
}
// (no NaN among the four)
__device__ __forceinline__ uint32_t e4m3_pack4_finite(float a, float b, float c, float d) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.0f), 448.0f),
                                                               fminf(fmaxf(b, -448.0f), 448.0f),
                                                               0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -448.0f), 448.0f),
                                                   fminf(fmaxf(d, -448.0f), 448.0f), (int)w,
                                                   true);
}
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  if ((a != a) | (b != b) | (c != c) | (d != d)) return e4m3_pack4_soft(a, b, c, d);
  return e4m3_pack4_finite(a, b, c, d);
}

// Four E2M1 codes in the low 16 bits (value q in bits 4 q ..): the hardware
// conversion at unit scale, which equals e2m1_code on every float32 input
// (NaN and infinities included; checked on the device as above).
__device__ __forceinline__ uint32_t e2m1_pack4(float a, float b, float c, float d) {
  uint32_t q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, c, d, 1.0f, 1);
  return q & 0xffffu;
}

// Element formats: exponent of the largest normal, code words per 32 values.
struct FmtE4M3 {
  static constexpr int EMAX = 8, WORDS = 8, BYTES = 32;
};
struct FmtE2M1 {
  static constexpr int EMAX = 2, WORDS = 4, BYTES = 16;
};

// Quantize 32 values: returns the scale code, writes F::WORDS little-endian
// words of element codes (E4M3: value i in byte i % 4 of word i / 4; E2M1:
// value i in bits 4 (i % 8) .. of word i / 8).
template <class F = FmtE4M3>
__device__ __forceinline__ uint32_t mx_quant32(const float* v, uint32_t* w) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent<F::EMAX>(amax);
  const float inv = mx_inv_scale(e);
  if constexpr (F::WORDS == 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = e4m3_pack4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv,
                        v[4 * i + 3] * inv);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = e2m1_pack4(v[8 * i] * inv, v[8 * i + 1] * inv, v[8 * i + 2] * inv,
                        v[8 * i + 3] * inv) |
             (e2m1_pack4(v[8 * i + 4] * inv, v[8 * i + 5] * inv, v[8 * i + 6] * inv,
                         v[8 * i + 7] * inv) << 16);
  }
  return (uint32_t)(e + 127);
}

}  // namespace moe
