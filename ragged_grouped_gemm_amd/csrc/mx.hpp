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
// Everything below is exact integer / power-of-two arithmetic on float32.
#pragma once

#include <stdint.h>

namespace moe {

// Shared exponent of a block from its largest magnitude (finite, >= 0).
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23) & 0xff;  // 0 for zero and float32 subnormals
  if (ef == 0) return -127;              // floor(log2 amax) <= -127 -> clamped
  const int e = ef - 127 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as a float32 (e in [-127, 119] for any finite float32 amax, so the
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

// Quantize 32 values: returns the scale code, writes 8 little-endian words of
// element codes (value i in byte i % 4 of word i / 4).
__device__ __forceinline__ uint32_t mx_quant32(const float* v, uint32_t* w) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  const float inv = mx_inv_scale(e);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t x = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) x |= e4m3_code(v[4 * i + q] * inv) << (8 * q);
    w[i] = x;
  }
  return (uint32_t)(e + 127);
}

}  // namespace moe
