// MXFP8 / MXFP4 quantizers (E4M3 or E2M1 elements, one E8M0 scale per 32):
// row copies, transposed weight copies and expert-segmented column copies.
// Code rows hold F::BYTES bytes per 32 elements (ld elements = ld * BYTES / 32
// bytes).
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

// The F::BYTES code bytes of one block (16-byte aligned).
template <class F>
__device__ __forceinline__ void store_block(uint8_t* dst, const uint32_t* w) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  d[0] = u32x4{w[0], w[1], w[2], w[3]};
  if constexpr (F::WORDS == 8) d[1] = u32x4{w[4], w[5], w[6], w[7]};
}

// Row copy: eight lanes per 32-block, four values per lane; a wave covers
// eight consecutive blocks (512 contiguous bytes of bf16 input).
template <class EL, class F>
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
    const int e = mx_exponent<F::EMAX>(amax);
    const float inv = mx_inv_scale(e);
    const long long ldb = ld / 32 * F::BYTES;
    if constexpr (F::WORDS == 8) {
      *reinterpret_cast<uint32_t*>(codes + r * ldb + 32 * b + 4 * sub) =
          e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    } else {
      *reinterpret_cast<uint16_t*>(codes + r * ldb + 16 * b + 2 * sub) =
          (uint16_t)e2m1_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
    if (sub == 0) scales[r * (ld / 32) + b] = (uint8_t)(e + 127);
  }
}

// Transposed copy of a batch [B, rows, n]: a workgroup quantizes one group of
// 32 rows for 256 columns, thread c holding column c (its 32 values come from
// 32 coalesced row reads of the workgroup) and writing 32 contiguous code
// bytes of output row b n + c.  (Weights only: made once, outside the layer.)
template <class EL, class F>
__global__ void __launch_bounds__(256)
    mx_transpose_kernel(const typename EL::storage* __restrict__ x, int n, int rows,
                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, long long ld,
                        long long ngroups) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  for (long long g = blockIdx.y; g < ngroups; g += gridDim.y) {
    const int nrb = rows / 32;
    const long long b = g / nrb;
    const int prow0 = (int)(g - b * nrb) * 32;
    if (c < n) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = ld1(x + (b * rows + prow0 + i) * n + c);
      uint32_t w[8];
      const uint32_t sc = mx_quant32<F>(v, w);
      store_block<F>(codes + (b * n + c) * (ld / 32 * F::BYTES) + prow0 / 32 * F::BYTES, w);
      scales[(b * n + c) * (ld / 32) + prow0 / 32] = (uint8_t)sc;
    }
  }
}

// Row and column copies of one group of 32 expert-ordered rows x 256 columns
// in one pass.  The workgroup copies the tile's raw 16-byte chunks (gathered
// rows) into LDS, row stride TILE_LD elements (bf16: 528 bytes, fp32: 1040,
// both 16 mod 256, so the 32 rows of a block read sit in distinct banks); the
// gate product is applied as values leave LDS.  Thread t then quantizes row
// t / 8 of 32-column block t % 8 into the row copy (so eight adjacent lanes
// write one row's 256 columns contiguously) and column t over the 32 rows into
// the column copy.  Staging the input type rather than float32
// halves the LDS of a bf16 workgroup, which doubles the workgroups a compute
// unit holds and so the loads in flight.
template <class S>
struct TileLd;
template <>
struct TileLd<uint16_t> {
  static constexpr int LD = 264;
};
template <>
struct TileLd<float> {
  static constexpr int LD = 260;
};

template <class EL, class F>
__global__ void __launch_bounds__(256)
    mx_rowcol_kernel(const typename EL::storage* __restrict__ x, int n, int E,
                     const int32_t* __restrict__ offsets, const int32_t* __restrict__ pad_offsets,
                     const int32_t* __restrict__ src_row, const int32_t* __restrict__ row_map,
                     const float* __restrict__ topk_w, int k, uint8_t* __restrict__ rcodes,
                     uint8_t* __restrict__ rscales, long long rld, uint8_t* __restrict__ ccodes,
                     uint8_t* __restrict__ cscales, long long cld, long long ngroups) {
  typedef typename EL::storage S;
  constexpr int V = EL::VEC;               // elements per 16-byte chunk
  constexpr int TLD = TileLd<S>::LD;
  __shared__ __attribute__((aligned(16))) S tile[32 * TLD];
  __shared__ long long s_src[32];
  __shared__ float s_w[32];
  __shared__ int s_row[32];                // routed row of tile row i (or -1)
  const int tid = threadIdx.x;
  // Workgroups are dealt round-robin over the 8 XCDs in launch order.  The
  // column copy of group g + 1 continues the 32-byte pieces of group g in the
  // same rows, so consecutive groups of one column chunk go to one XCD: its
  // L2 then merges the pieces into whole lines before they reach HBM.
  const int nb = gridDim.x * gridDim.y, n8 = nb & ~7;
  int vid = blockIdx.y * gridDim.x + blockIdx.x;
  if (vid < n8) vid = (vid & 7) * (n8 >> 3) + (vid >> 3);
  const int c0 = (vid / gridDim.y) * 256;
  for (long long g = vid % gridDim.y; g < ngroups; g += gridDim.y) {
    const int prow0 = (int)(g * 32);
    if (prow0 >= pad_offsets[E]) break;    // same for the whole workgroup
    int lo = 0, hi = E;                    // largest e with pad_offsets[e] <= prow0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pad_offsets[mid] <= prow0) lo = mid; else hi = mid;
    }
    if (tid < 32) {
      const int r = offsets[lo] + prow0 - pad_offsets[lo] + tid;
      const bool ok = r < offsets[lo + 1];
      const long long sr = ok ? (src_row ? (long long)src_row[r] : r) : -1;
      s_src[tid] = sr;
      s_row[tid] = ok ? r : -1;
      s_w[tid] = (ok && topk_w) ? row_gate(row_map, topk_w, k, sr, r) : 1.0f;
    }
    __syncthreads();
    // copy: 32 rows x 256 columns, one 16-byte chunk per thread per step
    constexpr int PER_ROW = 256 / V;                 // chunks per tile row
    constexpr int STEPS = 32 * PER_ROW / 256;
    u32x4 raw[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int idx = st * 256 + tid;
      const int i = idx / PER_ROW, cc = (idx % PER_ROW) * V;
      const long long sr = s_src[i];
      raw[st] = (sr >= 0 && c0 + cc < n)
                    ? *reinterpret_cast<const u32x4*>(x + sr * n + c0 + cc)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int idx = st * 256 + tid;
      const int i = idx / PER_ROW, cc = (idx % PER_ROW) * V;
      *reinterpret_cast<u32x4*>(tile + i * TLD + cc) = raw[st];
    }
    __syncthreads();
    float v[32];
    uint32_t w8[8];
    // row copy: row t / 8, block t % 8 (eight lanes write a row's 256 columns)
    {
      const int i = tid >> 3, b = tid & 7, col = c0 + 32 * b;
      const int r = s_row[i];
      if (rcodes && r >= 0 && col < n) {
        const float wi = s_w[i];
#pragma unroll
        for (int q = 0; q < 32 / V; ++q) {
          float t[V];
          unpack_chunk(*reinterpret_cast<const u32x4*>(tile + i * TLD + 32 * b + V * q), t, EL());
#pragma unroll
          for (int e = 0; e < V; ++e) v[V * q + e] = topk_w ? t[e] * wi : t[e];
        }
        const uint32_t sc = mx_quant32<F>(v, w8);
        store_block<F>(rcodes + (size_t)r * (rld / 32 * F::BYTES) + col / 32 * F::BYTES, w8);
        rscales[(size_t)r * (rld / 32) + col / 32] = (uint8_t)sc;
      }
    }
    // column copy: column t over the 32 rows
    if (ccodes && c0 + tid < n) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float t = ld1(tile + i * TLD + tid);
        v[i] = topk_w ? t * s_w[i] : t;
      }
      const uint32_t sc = mx_quant32<F>(v, w8);
      store_block<F>(ccodes + (size_t)(c0 + tid) * (cld / 32 * F::BYTES) + prow0 / 32 * F::BYTES,
                     w8);
      cscales[(size_t)(c0 + tid) * (cld / 32) + prow0 / 32] = (uint8_t)sc;
    }
    __syncthreads();
  }
}

// Decoded element values (exact in float32).  E4M3: (1 + m/8) 2^(e-7), or
// m 2^-9 for e = 0, NaN for S.1111.111; E2M1: (1 + m/2) 2^(e-1), or m/2.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if ((c & 0x7fu) == 0x7fu) v = __uint_as_float(0x7fc00000u);
  return (c & 0x80u) ? -v : v;
}
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float v = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 0x8u) ? -v : v;
}
// E8M0 scale 2^(s - 127) (s = 0 is the float32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// Unpermute-sum of MX rows: one wave per token, a lane per 16 elements (half
// a scale block): out[t] = sum_j w_j * decode(y[row_map[t, j]]) in float32 in
// slot order.  K > 0 fixes k at compile time (all k rows' loads of a unit in
// flight); K = 0 takes the run-time k.
template <class F, int K, bool BF_OUT>
__global__ void __launch_bounds__(256)
    combine_mx_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                      long long ld, const int32_t* __restrict__ row_map,
                      const float* __restrict__ w, int T, int R, int k_rt, int d,
                      void* __restrict__ out) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int k = K > 0 ? K : k_rt;
  const int units = d / 16;
  const long long ldb = ld / 32 * F::BYTES;                  // code bytes per row
  for (int u = lane; u < units; u += 64) {
    float acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
#pragma unroll(K > 0 ? K : 1)
    for (int j = 0; j < k; ++j) {
      int r = row_map[(size_t)t * k + j];
      r = (r < 0 || r >= R) ? 0 : r;
      const float wj = w ? w[(size_t)t * k + j] : 1.0f;
      const float sc = e8m0_value(scales[(size_t)r * (ld / 32) + u / 2]);
      float v[16];
      if constexpr (F::WORDS == 8) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(codes + (size_t)r * ldb + 16 * u);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = e4m3_value((c[q >> 2] >> (8 * (q & 3))) & 0xffu);
      } else {
        const u32x2 c = *reinterpret_cast<const u32x2*>(codes + (size_t)r * ldb + 8 * u);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = e2m1_value((c[q >> 3] >> (4 * (q & 7))) & 0xfu);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = fmaf(wj, v[q] * sc, acc[q]);
    }
    if constexpr (BF_OUT) {
      u32x4* o = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * d + 16 * u);
      o[0] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
      o[1] = u32x4{pack_bf16x2(acc[8], acc[9]), pack_bf16x2(acc[10], acc[11]),
                   pack_bf16x2(acc[12], acc[13]), pack_bf16x2(acc[14], acc[15])};
    } else {
      f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * d + 16 * u);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  }
}

template <class F, bool BF_OUT>
void launch_combine_mx(const moe_mx_t* y, const int32_t* row_map, const float* w, int T, int k,
                       int d, void* out, hipStream_t s) {
  const dim3 grid((T + 3) / 4);
  const int R = T * k;
#define MOE_CMX(KK)                                                                            \
  hipLaunchKernelGGL((combine_mx_kernel<F, KK, BF_OUT>), grid, dim3(256), 0, s, y->data,       \
                     y->scale, (long long)y->ld, row_map, w, T, R, k, d, out)
  switch (k) {
    case 1: MOE_CMX(1); break;
    case 2: MOE_CMX(2); break;
    case 4: MOE_CMX(4); break;
    case 8: MOE_CMX(8); break;
    default: MOE_CMX(0); break;
  }
#undef MOE_CMX
}

bool mx_ok(const moe_mx_t* m) {
  return m && m->data && m->scale && m->ld > 0 && m->ld % 32 == 0 && aligned16(m->data);
}

int grid_for(long long work, int per_block, int cap) {
  long long g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

template <class EL, class F>
void launch_rows(const void* x, long long rows, int n, const int32_t* src_row,
                 const int32_t* row_map, const float* topk_w, int k, const moe_mx_t* out,
                 hipStream_t s) {
  const long long blocks = rows * (n / 32);
  hipLaunchKernelGGL((mx_rows_kernel<EL, F>), dim3(grid_for(blocks, 32, 16384)), dim3(256), 0, s,
                     reinterpret_cast<const typename EL::storage*>(x), rows, n, src_row, row_map,
                     topk_w, k, out->data, out->scale, (long long)out->ld);
}

template <class EL, class F>
void launch_transpose(const void* x, int n, int rows, const moe_mx_t* out, long long ngroups,
                      hipStream_t s) {
  const int gx = (n + 255) / 256;
  const int gy = (int)(ngroups > 16384 ? 16384 : ngroups);
  hipLaunchKernelGGL((mx_transpose_kernel<EL, F>), dim3(gx, gy), dim3(256), 0, s,
                     reinterpret_cast<const typename EL::storage*>(x), n, rows, out->data,
                     out->scale, (long long)out->ld, ngroups);
}

template <class EL, class F>
void launch_rowcol(const void* x, int n, int E, const int32_t* offsets, const int32_t* pad_offsets,
                   const int32_t* src_row, const int32_t* row_map, const float* topk_w, int k,
                   const moe_mx_t* row_out, const moe_mx_t* col_out, long long ngroups,
                   hipStream_t s) {
  const int gx = (n + 255) / 256;
  const int gy = (int)(ngroups > 16384 ? 16384 : ngroups);
  hipLaunchKernelGGL((mx_rowcol_kernel<EL, F>), dim3(gx, gy), dim3(256), 0, s,
                     reinterpret_cast<const typename EL::storage*>(x), n, E, offsets, pad_offsets,
                     src_row, row_map, topk_w, k, row_out ? row_out->data : nullptr,
                     row_out ? row_out->scale : nullptr, row_out ? (long long)row_out->ld : 0LL,
                     col_out->data, col_out->scale, (long long)col_out->ld, ngroups);
}

}  // namespace

template <class F>
moe_status_t mx_quantize_impl(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                             void* stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && rows >= 0 && n > 0 && n % 32 == 0);
  MOE_CHECK_ARG(mx_ok(out) && out->ld >= n);
  MOE_CHECK_ARG(rows == 0 || (x && aligned16(x)));
  if (rows == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MOE_BF16) launch_rows<BF16, F>(x, rows, n, nullptr, nullptr, nullptr, 0, out, s);
  else launch_rows<F32, F>(x, rows, n, nullptr, nullptr, nullptr, 0, out, s);
  return launch_status();
}

template <class F>
moe_status_t mx_quantize_transpose_impl(const void* x, int dtype, int batches, int rows, int n,
                                       moe_mx_t* out, void* stream) {
  MOE_CHECK_ARG(valid_dtype(dtype) && batches >= 0 && rows >= 0 && rows % 32 == 0 && n > 0);
  MOE_CHECK_ARG(mx_ok(out) && out->ld >= rows);
  const long long groups = (long long)batches * (rows / 32);
  MOE_CHECK_ARG(groups == 0 || (x && aligned16(x)));
  if (groups == 0) return MOE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MOE_BF16) launch_transpose<BF16, F>(x, n, rows, out, groups, s);
  else launch_transpose<F32, F>(x, n, rows, out, groups, s);
  return launch_status();
}

template <class F>
moe_status_t mx_quantize_experts_impl(const void* x, int dtype, const int32_t* src_row,
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
  if (col_out) {
    // both copies from one read of the rows
    const long long groups = moe_mx_col_len(R, E) / 32;
    if (bf)
      launch_rowcol<BF16, F>(x, n, E, offsets, pad_offsets, src_row, row_map, topk_w, k, row_out,
                             col_out, groups, s);
    else
      launch_rowcol<F32, F>(x, n, E, offsets, pad_offsets, src_row, row_map, topk_w, k, row_out,
                            col_out, groups, s);
  } else if (bf) {
    launch_rows<BF16, F>(x, R, n, src_row, row_map, topk_w, k, row_out, s);
  } else {
    launch_rows<F32, F>(x, R, n, src_row, row_map, topk_w, k, row_out, s);
  }
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_mx_col_len(int R, int E) {
  const int64_t n = (int64_t)R + 31 * (int64_t)E;
  return (n + 127) / 128 * 128;
}

int64_t moe_mx_col_ld(int R, int E, int dtype) {
  if (dtype != MOE_E4M3 && dtype != MOE_E2M1) return 0;
  const int64_t unit = dtype == MOE_E2M1 ? 256 : 128;  // elements per 128 bytes
  int64_t lines = (moe_mx_col_len(R, E) + unit - 1) / unit;
  if (lines % 2 == 0) ++lines;
  return lines * unit;
}

moe_status_t moe_mx_quantize(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                             void* stream) {
  return mx_quantize_impl<FmtE4M3>(x, dtype, rows, n, out, stream);
}
moe_status_t moe_mxfp4_quantize(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                                void* stream) {
  return mx_quantize_impl<FmtE2M1>(x, dtype, rows, n, out, stream);
}
moe_status_t moe_mx_quantize_transpose(const void* x, int dtype, int batches, int rows, int n,
                                       moe_mx_t* out, void* stream) {
  return mx_quantize_transpose_impl<FmtE4M3>(x, dtype, batches, rows, n, out, stream);
}
moe_status_t moe_mxfp4_quantize_transpose(const void* x, int dtype, int batches, int rows, int n,
                                          moe_mx_t* out, void* stream) {
  return mx_quantize_transpose_impl<FmtE2M1>(x, dtype, batches, rows, n, out, stream);
}
moe_status_t moe_mx_quantize_experts(const void* x, int dtype, const int32_t* src_row,
                                     const int32_t* row_map, const float* topk_w, int k,
                                     const int32_t* offsets, const int32_t* pad_offsets, int E,
                                     int R, int n, moe_mx_t* row_out, moe_mx_t* col_out,
                                     void* stream) {
  return mx_quantize_experts_impl<FmtE4M3>(x, dtype, src_row, row_map, topk_w, k, offsets,
                                           pad_offsets, E, R, n, row_out, col_out, stream);
}
moe_status_t moe_mxfp4_quantize_experts(const void* x, int dtype, const int32_t* src_row,
                                        const int32_t* row_map, const float* topk_w, int k,
                                        const int32_t* offsets, const int32_t* pad_offsets, int E,
                                        int R, int n, moe_mx_t* row_out, moe_mx_t* col_out,
                                        void* stream) {
  return mx_quantize_experts_impl<FmtE2M1>(x, dtype, src_row, row_map, topk_w, k, offsets,
                                           pad_offsets, E, R, n, row_out, col_out, stream);
}

moe_status_t moe_unpermute_combine_mx(const moe_mx_t* y, int y_dtype, const int32_t* row_map,
                                      const float* topk_w, int T, int k, int d, void* out,
                                      int out_dtype, void* stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && d > 0 && d % 32 == 0);
  MOE_CHECK_ARG(y_dtype == MOE_E4M3 || y_dtype == MOE_E2M1);
  MOE_CHECK_ARG(out_dtype == MOE_BF16 || out_dtype == MOE_F32);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(mx_ok(y) && y->ld >= d && row_map && out && aligned16(out));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = out_dtype == MOE_BF16;
  if (y_dtype == MOE_E4M3) {
    if (bf) launch_combine_mx<FmtE4M3, true>(y, row_map, topk_w, T, k, d, out, s);
    else launch_combine_mx<FmtE4M3, false>(y, row_map, topk_w, T, k, d, out, s);
  } else {
    if (bf) launch_combine_mx<FmtE2M1, true>(y, row_map, topk_w, T, k, d, out, s);
    else launch_combine_mx<FmtE2M1, false>(y, row_map, topk_w, T, k, d, out, s);
  }
  return launch_status();
}

}  // extern "C"
