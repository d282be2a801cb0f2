// MXFP8 quantizers (E4M3 elements, one E8M0 scale per 32): row copies,
// transposed weight copies and expert-segmented column copies.
//
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上", section
// "MXFP8 および NVFP4 量子化の融合による露出メモリオーバーヘッドの削減": GEMM
// operands in MXFP8 with a transposed copy for the backward pass; the
// quantizers here read their values straight from the source rows (the token
// gather of the permute, or the gate product of the combine backward), so no
// bf16 intermediate is written.  The element and scale rule is in mx.hpp.
#include "common.hpp"
#include "mx.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float ld1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }

// Gate of routed row r (token t): topk_w[t k + j] for the slot j with
// row_map[t k + j] == r.
__device__ __forceinline__ float row_gate(const int32_t* __restrict__ row_map,
                                          const float* __restrict__ topk_w, int k, long long t,
                                          int r) {
  float w = 0.0f;
  for (int j = 0; j < k; ++j)
    if (row_map[t * k + j] == r) w = topk_w[t * k + j];
  return w;
}

// Row copy: eight lanes per 32-block, four values per lane; a wave covers
// eight consecutive blocks (512 contiguous bytes of bf16 input).
template <class EL>
__global__ void __launch_bounds__(256)
    mx_rows_kernel(const typename EL::storage* __restrict__ x, long long rows, int n,
                   const int32_t* __restrict__ src_row, const int32_t* __restrict__ row_map,
                   const float* __restrict__ topk_w, int k, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales, long long ld) {
  const int nb = n / 32;
  const long long total = rows * nb;
  const int sub = threadIdx.x & 7;
  const long long stride = ((long long)gridDim.x * blockDim.x) >> 3;
  for (long long blk = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 3; blk < total;
       blk += stride) {
    const long long r = blk / nb;
    const int b = (int)(blk - r * nb);
    const long long sr = src_row ? (long long)src_row[r] : r;
    float v[4];
    load4(x + sr * n + 32 * b + 4 * sub, v);
    if (topk_w) {
      const float w = row_gate(row_map, topk_w, k, sr, (int)r);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] *= w;
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    // the eight lanes of a block are aligned groups of eight: xor 1, 2, 4 stay inside
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    const int e = mx_exponent(amax);
    const float inv = mx_inv_scale(e);
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) word |= e4m3_code(v[q] * inv) << (8 * q);
    *reinterpret_cast<uint32_t*>(codes + r * ld + 32 * b + 4 * sub) = word;
    if (sub == 0) scales[r * (ld / 32) + b] = (uint8_t)(e + 127);
  }
}

enum { COLS_SEGMENTS = 0, COLS_TRANSPOSE = 1 };

// Column copies: a workgroup quantizes one group of 32 source rows for 256
// columns, thread c holding column c (its 32 values come from 32 coalesced
// row reads of the workgroup) and writing 32 contiguous code bytes.
//  COLS_SEGMENTS: group g = tokens [32 g, 32 g + 32) of the padded expert
//    segments; source row of token position p in segment e is
//    src_row[offsets[e] + p - pad_offsets[e]] (zero past the segment end).
//  COLS_TRANSPOSE: group g = rows [32 rb, 32 rb + 32) of matrix b of a batch
//    [B, rows, n]; output row b n + c.
template <class EL, int MODE>
__global__ void __launch_bounds__(256)
    mx_cols_kernel(const typename EL::storage* __restrict__ x, int n, int rows, int E,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ pad_offsets,
                   const int32_t* __restrict__ src_row, const int32_t* __restrict__ row_map,
                   const float* __restrict__ topk_w, int k, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales, long long ld, long long ngroups) {
  __shared__ long long s_src[32];
  __shared__ float s_w[32];
  const int tid = threadIdx.x;
  const int c = blockIdx.x * 256 + tid;
  for (long long g = blockIdx.y; g < ngroups; g += gridDim.y) {
    long long out_base;
    int prow0;
    if constexpr (MODE == COLS_SEGMENTS) {
      prow0 = (int)(g * 32);
      if (prow0 >= pad_offsets[E]) break;  // same for the whole workgroup
      int lo = 0, hi = E;                  // largest e with pad_offsets[e] <= prow0
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pad_offsets[mid] <= prow0) lo = mid; else hi = mid;
      }
      if (tid < 32) {
        const int r = offsets[lo] + prow0 - pad_offsets[lo] + tid;
        const bool ok = r < offsets[lo + 1];
        const long long sr = ok ? (src_row ? (long long)src_row[r] : r) : -1;
        s_src[tid] = sr;
        s_w[tid] = (ok && topk_w) ? row_gate(row_map, topk_w, k, sr, r) : 1.0f;
      }
      out_base = 0;
    } else {
      const int nrb = rows / 32;
      const long long b = g / nrb;
      prow0 = (int)(g - b * nrb) * 32;
      if (tid < 32) {
        s_src[tid] = b * rows + prow0 + tid;
        s_w[tid] = 1.0f;
      }
      out_base = b * n;
    }
    __syncthreads();
    if (c < n) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const long long sr = s_src[i];
        float t = sr >= 0 ? ld1(x + sr * n + c) : 0.0f;
        if (topk_w) t *= s_w[i];
        v[i] = t;
      }
      uint32_t w[8];
      const uint32_t sc = mx_quant32(v, w);
      u32x4* dst = reinterpret_cast<u32x4*>(codes + (out_base + c) * ld + prow0);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
      scales[(out_base + c) * (ld / 32) + prow0 / 32] = (uint8_t)sc;
    }
    __syncthreads();
  }
}

bool mx_ok(const moe_mx_t* m) {
  return m && m->data && m->scale && m->ld > 0 && m->ld % 32 == 0 && aligned16(m->data);
}

int grid_for(long long work, int per_block, int cap) {
  long long g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

template <class EL>
void launch_rows(const void* x, long long rows, int n, const int32_t* src_row,
                 const int32_t* row_map, const float* topk_w, int k, const moe_mx_t* out,
                 hipStream_t s) {
  const long long blocks = rows * (n / 32);
  hipLaunchKernelGGL(mx_rows_kernel<EL>, dim3(grid_for(blocks, 32, 16384)), dim3(256), 0, s,
                     reinterpret_cast<const typename EL::storage*>(x), rows, n, src_row, row_map,
                     topk_w, k, out->data, out->scale, (long long)out->ld);
}

template <class EL, int MODE>
void launch_cols(const void* x, int n, int rows, int E, const int32_t* offsets,
                 const int32_t* pad_offsets, const int32_t* src_row, const int32_t* row_map,
                 const float* topk_w, int k, const moe_mx_t* out, long long ngroups,
                 hipStream_t s) {
  const int gx = (n + 255) / 256;
  const int gy = (int)(ngroups < 1 ? 1 : (ngroups > 16384 ? 16384 : ngroups));
  hipLaunchKernelGGL((mx_cols_kernel<EL, MODE>), dim3(gx, gy), dim3(256), 0, s,
                     reinterpret_cast<const typename EL::storage*>(x), n, rows, E, offsets,
                     pad_offsets, src_row, row_map, topk_w, k, out->data, out->scale,
                     (long long)out->ld, ngroups);
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_mx_col_len(int R, int E) {
  const int64_t n = (int64_t)R + 31 * (int64_t)E;
  return (n + 127) / 128 * 128;
}

moe_status_t moe_mx_quantize(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                             void* stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && rows >= 0 && n > 0 && n % 32 == 0);
  MOE_CHECK_ARG(mx_ok(out) && out->ld >= n);
  MOE_CHECK_ARG(rows == 0 || (x && aligned16(x)));
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MOE_BF16) launch_rows<BF16>(x, rows, n, nullptr, nullptr, nullptr, 0, out, s);
  else launch_rows<F32>(x, rows, n, nullptr, nullptr, nullptr, 0, out, s);
  return launch_status();
}

moe_status_t moe_mx_quantize_transpose(const void* x, int dtype, int batches, int rows, int n,
                                       moe_mx_t* out, void* stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && batches >= 0 && rows >= 0 && rows % 32 == 0 && n > 0);
  MOE_CHECK_ARG(mx_ok(out) && out->ld >= rows);
  const long long groups = (long long)batches * (rows / 32);
  MOE_CHECK_ARG(groups == 0 || (x && aligned16(x)));
  if (groups == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MOE_BF16)
    launch_cols<BF16, COLS_TRANSPOSE>(x, n, rows, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      0, out, groups, s);
  else
    launch_cols<F32, COLS_TRANSPOSE>(x, n, rows, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     0, out, groups, s);
  return launch_status();
}

moe_status_t moe_mx_quantize_experts(const void* x, int dtype, const int32_t* src_row,
                                     const int32_t* row_map, const float* topk_w, int k,
                                     const int32_t* offsets, const int32_t* pad_offsets, int E,
                                     int R, int n, moe_mx_t* row_out, moe_mx_t* col_out,
                                     void* stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && R >= 0 && n > 0 && n % 32 == 0);
  MOE_CHECK_ARG(E >= 1 && E <= MOE_MAX_EXPERTS);
  MOE_CHECK_ARG((row_map == nullptr) == (topk_w == nullptr));
  MOE_CHECK_ARG(topk_w == nullptr || (src_row && k >= 1 && k <= MOE_MAX_TOPK));
  MOE_CHECK_ARG(row_out || col_out);
  MOE_CHECK_ARG(!row_out || (mx_ok(row_out) && row_out->ld >= n));
  MOE_CHECK_ARG(!col_out || (mx_ok(col_out) && col_out->ld >= moe_mx_col_len(R, E) &&
                             offsets && pad_offsets));
  MOE_CHECK_ARG(R == 0 || (x && aligned16(x)));
  if (R == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = dtype == MOE_BF16;
  if (row_out) {
    if (bf) launch_rows<BF16>(x, R, n, src_row, row_map, topk_w, k, row_out, s);
    else launch_rows<F32>(x, R, n, src_row, row_map, topk_w, k, row_out, s);
  }
  if (col_out) {
    const long long groups = moe_mx_col_len(R, E) / 32;
    if (bf)
      launch_cols<BF16, COLS_SEGMENTS>(x, n, 0, E, offsets, pad_offsets, src_row, row_map,
                                       topk_w, k, col_out, groups, s);
    else
      launch_cols<F32, COLS_SEGMENTS>(x, n, 0, E, offsets, pad_offsets, src_row, row_map, topk_w,
                                      k, col_out, groups, s);
  }
  return launch_status();
}

}  // extern "C"
