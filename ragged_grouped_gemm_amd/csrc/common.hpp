// Shared helpers of the gfx950 kernels: element conversions, vector types,
// host-side argument checks and launch bookkeeping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element traits: storage type, elements per 16-byte chunk.
struct BF16 {
  typedef uint16_t storage;
  static constexpr int VEC = 8;
};
struct F32 {
  typedef float storage;
  static constexpr int VEC = 4;
};

// Load 4 consecutive elements as float.
__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
  u32x2 w = *reinterpret_cast<const u32x2*>(p);
  v[0] = bf16_bits_to_f32(w[0] & 0xffffu);
  v[1] = bf16_bits_to_f32(w[0] >> 16);
  v[2] = bf16_bits_to_f32(w[1] & 0xffffu);
  v[3] = bf16_bits_to_f32(w[1] >> 16);
}
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  f32x4 w = *reinterpret_cast<const f32x4*>(p);
  v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
}
// Store 4 consecutive elements (rounded to the storage type).
__device__ __forceinline__ void store4(uint16_t* p, const float v[4]) {
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  f32x4 w = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = w;
}

// Unpack a 16-byte chunk into floats (8 bf16 or 4 f32).
__device__ __forceinline__ void unpack_chunk(const u32x4& c, float* v, BF16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(c[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(c[i] >> 16);
  }
}
__device__ __forceinline__ void unpack_chunk(const u32x4& c, float* v, F32) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(c[i]);
}
__device__ __forceinline__ u32x4 pack_chunk(const float* v, BF16) {
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  return c;
}
__device__ __forceinline__ u32x4 pack_chunk(const float* v, F32) {
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(v[i]);
  return c;
}

// ----------------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
  // Fixed butterfly order: the result is identical on every lane and run.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void set_err(int32_t* err_word, uint32_t bits) {
  if (err_word) atomicOr(reinterpret_cast<unsigned int*>(err_word), bits);
}

// ----------------------------------------------------------------- host side

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline moe_status_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

inline size_t dtype_size(int dtype) { return dtype == MOE_F32 ? 4 : 2; }
inline bool valid_dtype(int dtype) { return dtype == MOE_F32 || dtype == MOE_BF16; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// db[e][n] = column sums of g [R, N] over the rows of expert segment e
// (float32; added to db when accumulate).
moe_status_t launch_segment_colsum(int dtype, const void* g, const int32_t* offsets, int E,
                                   int R, int N, float* db, int accumulate, hipStream_t s);

}  // namespace moe

#define MOE_CHECK_ARG(cond)                 \
  do {                                      \
    if (!(cond)) return MOE_ERR_INVALID_ARG; \
  } while (0)
