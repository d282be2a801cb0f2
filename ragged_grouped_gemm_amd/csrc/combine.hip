// Weighted unpermute / combine and its backward.
//
// out[t] = sum_{j<k} w[t,j] * y[row_map[t,j]]: the gate-weighted sum of a
// token's k expert outputs, accumulated in float32 in slot order and rounded
// once.  The backward scatters w[t,j] * dout[t] to the rows and takes the dot
// products <dout[t], y[row]> for the gate gradient.  Both are HBM-bound
// gathers: one wave per token, 16-byte vectors along d, no atomics (each row
// belongs to exactly one (t, j)), so results are deterministic.
#include "common.hpp"

namespace moe {

template <class EL>
__global__ void __launch_bounds__(256) combine_kernel(const u32x4* __restrict__ y,
                                                      const int32_t* __restrict__ row_map,
                                                      const float* __restrict__ w, int T, int k,
                                                      int R, int chunks, u32x4* __restrict__ out) {
  constexpr int V = EL::VEC;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int lane = threadIdx.x & 63;
  int rows[MOE_MAX_TOPK];
  float ws[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    int r = row_map[(size_t)t * k + j];
    rows[j] = (r < 0 || r >= R) ? 0 : r;
    ws[j] = w ? w[(size_t)t * k + j] : 1.0f;
  }
  for (int c = lane; c < chunks; c += 64) {
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
    for (int j = 0; j < k; ++j) {
      float v[V];
      unpack_chunk(y[(size_t)rows[j] * chunks + c], v, EL());
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = fmaf(ws[j], v[q], acc[q]);
    }
    out[(size_t)t * chunks + c] = pack_chunk(acc, EL());
  }
}

template <class EL>
__global__ void __launch_bounds__(256) combine_bwd_kernel(
    const u32x4* __restrict__ dout, const u32x4* __restrict__ y,
    const int32_t* __restrict__ row_map, const float* __restrict__ w, int T, int k, int R,
    int chunks, u32x4* __restrict__ dy, float* __restrict__ dw) {
  constexpr int V = EL::VEC;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int lane = threadIdx.x & 63;
  for (int j = 0; j < k; ++j) {
    int r = row_map[(size_t)t * k + j];
    r = (r < 0 || r >= R) ? 0 : r;
    const float wj = w ? w[(size_t)t * k + j] : 1.0f;
    float part = 0.0f;
    for (int c = lane; c < chunks; c += 64) {
      float g[V], v[V], o[V];
      unpack_chunk(dout[(size_t)t * chunks + c], g, EL());
      if (dw) unpack_chunk(y[(size_t)r * chunks + c], v, EL());
#pragma unroll
      for (int q = 0; q < V; ++q) {
        if (dw) part = fmaf(g[q], v[q], part);
        o[q] = wj * g[q];
      }
      if (dy) dy[(size_t)r * chunks + c] = pack_chunk(o, EL());
    }
    float tot = wave_sum(part);
    if (lane == 0 && dw) dw[(size_t)t * k + j] = tot;
  }
}

// The same two kernels for a compile-time k: a lane issues the loads of all k
// rows of a chunk (and, backward, reads d_out once) before using any, so each
// lane keeps k + 1 loads in flight.  Sums run in the same order as above, so
// the results are identical.
// 16-byte global access, optionally with the nontemporal hint.  The combine
// and the unpermute-sum stream their inputs (every routed row is read once)
// and outputs (read by no later kernel of the layer) with it: measured 8 %
// and 16 % faster at dsv3_fwdbwd.  The combine backward writes dY, which
// the next GEMMs read, so it keeps the default policy.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, const u32x4& v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <class EL, int K>
__global__ void __launch_bounds__(256) combine_kernel_k(const u32x4* __restrict__ y,
                                                        const int32_t* __restrict__ row_map,
                                                        const float* __restrict__ w, int T, int R,
                                                        int chunks, u32x4* __restrict__ out) {
  constexpr int V = EL::VEC;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int rows[K];
  float ws[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = row_map[(size_t)t * K + j];
    rows[j] = (r < 0 || r >= R) ? 0 : r;
    ws[j] = w ? w[(size_t)t * K + j] : 1.0f;
  }
  for (int c = lane; c < chunks; c += 64) {
    u32x4 raw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = ld16<true>(y + (size_t)rows[j] * chunks + c);
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float v[V];
      unpack_chunk(raw[j], v, EL());
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = fmaf(ws[j], v[q], acc[q]);
    }
    st16<true>(out + (size_t)t * chunks + c, pack_chunk(acc, EL()));
  }
}

template <class EL, int K>
__global__ void __launch_bounds__(256) combine_bwd_kernel_k(
    const u32x4* __restrict__ dout, const u32x4* __restrict__ y,
    const int32_t* __restrict__ row_map, const float* __restrict__ w, int T, int R, int chunks,
    u32x4* __restrict__ dy, float* __restrict__ dw) {
  constexpr int V = EL::VEC;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int rows[K];
  float ws[K], part[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int r = row_map[(size_t)t * K + j];
    rows[j] = (r < 0 || r >= R) ? 0 : r;
    ws[j] = w ? w[(size_t)t * K + j] : 1.0f;
    part[j] = 0.0f;
  }
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 graw = dout[(size_t)t * chunks + c];
    u32x4 raw[K];
    if (dw) {
#pragma unroll
      for (int j = 0; j < K; ++j) raw[j] = y[(size_t)rows[j] * chunks + c];
    }
    float g[V];
    unpack_chunk(graw, g, EL());
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (dw) {
        float v[V];
        unpack_chunk(raw[j], v, EL());
#pragma unroll
        for (int q = 0; q < V; ++q) part[j] = fmaf(g[q], v[q], part[j]);
      }
      if (dy) {
        float o[V];
#pragma unroll
        for (int q = 0; q < V; ++q) o[q] = ws[j] * g[q];
        dy[(size_t)rows[j] * chunks + c] = pack_chunk(o, EL());
      }
    }
  }
  if (dw) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float tot = wave_sum(part[j]);
      if (lane == 0) dw[(size_t)t * K + j] = tot;
    }
  }
}

// Bias gradient of a grouped linear map: db[e][n] = sum over the rows of
// segment e of g[r][n], float32 (added to db when `accumulate`).
// grid: (ceil(N / CS_COLS), E), 1024 threads.  A block owns CS_COLS columns
// of one expert; a lane owns one 16-byte chunk (V columns) of every CS_RPW-th
// row of the wave's share, the 16 waves take interleaved groups of CS_RPW rows,
// so the segment is read in whole 128-byte pieces by the whole block at once
// (the sum is HBM-bound, not latency-bound, even for a 16K-row expert).  The
// partial sums are combined in a fixed order -- a butterfly over the row
// slots of a wave, then the waves in order -- so the result does not depend
// on timing.
static constexpr int CS_LPR = 8;                  // lanes per row (8 x 16 bytes)
static constexpr int CS_RPW = 64 / CS_LPR;        // rows per wave instruction
static constexpr int CS_WAVES = 16;

template <class EL>
__global__ void __launch_bounds__(1024) segment_colsum_kernel(const typename EL::storage* g,
                                                              const int32_t* __restrict__ offsets,
                                                              int R, int N, float* db,
                                                              int accumulate) {
  constexpr int V = EL::VEC;
  constexpr int COLS = CS_LPR * V;
  __shared__ float part[CS_WAVES][COLS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane % CS_LPR, slot = lane / CS_LPR;
  const int e = blockIdx.y;
  const int col = blockIdx.x * COLS + c * V;
  const int s = min(max(offsets[e], 0), R), t = min(max(offsets[e + 1], s), R);
  float acc[V], acc2[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = acc2[q] = 0.0f;
  if (col < N) {
    const u32x4* src = reinterpret_cast<const u32x4*>(g + col);
    const size_t ld = (size_t)N * sizeof(typename EL::storage) / 16;   // row stride in chunks
    constexpr int STEP = CS_WAVES * CS_RPW;
    int r = s + w * CS_RPW + slot;
    // two rows in flight per lane, summed into two accumulators in a fixed order
    for (; r + STEP < t; r += 2 * STEP) {
      const u32x4 a = src[(size_t)r * ld], b = src[(size_t)(r + STEP) * ld];
      float va[V], vb[V];
      unpack_chunk(a, va, EL());
      unpack_chunk(b, vb, EL());
#pragma unroll
      for (int q = 0; q < V; ++q) {
        acc[q] += va[q];
        acc2[q] += vb[q];
      }
    }
    if (r < t) {
      float va[V];
      unpack_chunk(src[(size_t)r * ld], va, EL());
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += va[q];
    }
  }
#pragma unroll
  for (int q = 0; q < V; ++q) {
    float v = acc[q] + acc2[q];
    // the row slots of the wave: lanes that differ in bits 3..5
#pragma unroll
    for (int o = CS_LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    acc[q] = v;
  }
  if (slot == 0) {
#pragma unroll
    for (int q = 0; q < V; ++q) part[w][c * V + q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < COLS) {
    const int n = blockIdx.x * COLS + threadIdx.x;
    if (n < N) {
      float tot = 0.0f;
#pragma unroll
      for (int i = 0; i < CS_WAVES; ++i) tot += part[i][threadIdx.x];
      float* o = db + (size_t)e * N + n;
      *o = accumulate ? *o + tot : tot;
    }
  }
}

template __global__ void segment_colsum_kernel<BF16>(const uint16_t*, const int32_t*, int, int,
                                                     float*, int);
template __global__ void segment_colsum_kernel<F32>(const float*, const int32_t*, int, int, float*,
                                                    int);

moe_status_t launch_segment_colsum(int dtype, const void* g, const int32_t* offsets, int E,
                                   int R, int N, float* db, int accumulate, hipStream_t s) {
  // N is a multiple of 8, so rows are whole 16-byte chunks (bf16 and float32)
  const int cols = CS_LPR * (dtype == MOE_BF16 ? BF16::VEC : F32::VEC);
  dim3 grid((N + cols - 1) / cols, E);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(segment_colsum_kernel<BF16>, grid, dim3(64 * CS_WAVES), 0, s,
                       reinterpret_cast<const uint16_t*>(g), offsets, R, N, db, accumulate);
  else
    hipLaunchKernelGGL(segment_colsum_kernel<F32>, grid, dim3(64 * CS_WAVES), 0, s,
                       reinterpret_cast<const float*>(g), offsets, R, N, db, accumulate);
  return launch_status();
}

// Row permutation of the FC1 weights between canonical and packed layouts.
// Canonical row i < f (gate) <-> packed 2G*(i/G) + i%G; row f+i (linear) <->
// packed 2G*(i/G) + G + i%G.  One wave per row; 16-byte copies.
__device__ __forceinline__ int packed_row(int i, int f, int G) {
  if (i < f) return 2 * G * (i / G) + i % G;
  i -= f;
  return 2 * G * (i / G) + G + i % G;
}

__global__ void __launch_bounds__(256) repack_kernel(const u32x4* __restrict__ w,
                                                     const float* __restrict__ b, int E, int f,
                                                     int G, int chunks, int inverse,
                                                     u32x4* __restrict__ wo,
                                                     float* __restrict__ bo) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // global row over E * 2f
  int lane = threadIdx.x & 63;
  if (row >= E * 2 * f) return;
  int e = row / (2 * f), i = row % (2 * f);
  int p = packed_row(i, f, G);
  int src = inverse ? p : i, dst = inverse ? i : p;
  const u32x4* s = w + ((size_t)e * 2 * f + src) * chunks;
  u32x4* d = wo + ((size_t)e * 2 * f + dst) * chunks;
  for (int c = lane; c < chunks; c += 64) d[c] = s[c];
  if (b && lane == 0) bo[(size_t)e * 2 * f + dst] = b[(size_t)e * 2 * f + src];
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_glu_granularity(void) { return 32; }

moe_status_t moe_unpermute_combine(const void* y, int dtype, const int32_t* row_map,
                                   const float* topk_w, int T, int k, int d, void* out,
                                   void* stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && d > 0 && valid_dtype(dtype));
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(y && row_map && out && aligned16(y) && aligned16(out));
  MOE_CHECK_ARG((d * dtype_size(dtype)) % 16 == 0);
  int chunks = (int)(d * dtype_size(dtype) / 16);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((T + 3) / 4);
  const u32x4* yy = reinterpret_cast<const u32x4*>(y);
  u32x4* oo = reinterpret_cast<u32x4*>(out);
  const bool bf = dtype == MOE_BF16;
#define MOE_COMBINE_K(KK)                                                                  \
  case KK:                                                                                 \
    if (bf)                                                                                \
      hipLaunchKernelGGL((combine_kernel_k<BF16, KK>), grid, dim3(256), 0, s, yy, row_map, \
                         topk_w, T, T * k, chunks, oo);                                    \
    else                                                                                   \
      hipLaunchKernelGGL((combine_kernel_k<F32, KK>), grid, dim3(256), 0, s, yy, row_map,  \
                         topk_w, T, T * k, chunks, oo);                                    \
    return launch_status();
  switch (k) {
    MOE_COMBINE_K(1)
    MOE_COMBINE_K(2)
    MOE_COMBINE_K(4)
    MOE_COMBINE_K(8)
    default:
      break;
  }
#undef MOE_COMBINE_K
  if (bf)
    hipLaunchKernelGGL(combine_kernel<BF16>, grid, dim3(256), 0, s, yy, row_map, topk_w, T, k,
                       T * k, chunks, oo);
  else
    hipLaunchKernelGGL(combine_kernel<F32>, grid, dim3(256), 0, s, yy, row_map, topk_w, T, k,
                       T * k, chunks, oo);
  return launch_status();
}

moe_status_t moe_unpermute_combine_bwd(const void* d_out, const void* y, int dtype,
                                       const int32_t* row_map, const float* topk_w, int T,
                                       int k, int d, void* d_y, float* d_topk_w, void* stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && d > 0 && valid_dtype(dtype));
  if (T == 0) return MOE_OK;
  // unit weights when topk_w is NULL; y is read only for d_topk_w
  MOE_CHECK_ARG(d_out && row_map && (d_y || d_topk_w) && (y || !d_topk_w));
  MOE_CHECK_ARG(aligned16(d_out) && aligned16(y) && aligned16(d_y));
  MOE_CHECK_ARG((d * dtype_size(dtype)) % 16 == 0);
  int chunks = (int)(d * dtype_size(dtype) / 16);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((T + 3) / 4);
  const u32x4* gg = reinterpret_cast<const u32x4*>(d_out);
  const u32x4* yy = reinterpret_cast<const u32x4*>(y);
  u32x4* dd = reinterpret_cast<u32x4*>(d_y);
  const bool bf = dtype == MOE_BF16;
#define MOE_COMBINE_BWD_K(KK)                                                                 \
  case KK:                                                                                    \
    if (bf)                                                                                   \
      hipLaunchKernelGGL((combine_bwd_kernel_k<BF16, KK>), grid, dim3(256), 0, s, gg, yy,     \
                         row_map, topk_w, T, T * k, chunks, dd, d_topk_w);                    \
    else                                                                                      \
      hipLaunchKernelGGL((combine_bwd_kernel_k<F32, KK>), grid, dim3(256), 0, s, gg, yy,      \
                         row_map, topk_w, T, T * k, chunks, dd, d_topk_w);                    \
    return launch_status();
  switch (k) {
    MOE_COMBINE_BWD_K(1)
    MOE_COMBINE_BWD_K(2)
    MOE_COMBINE_BWD_K(4)
    MOE_COMBINE_BWD_K(8)
    default:
      break;
  }
#undef MOE_COMBINE_BWD_K
  if (bf)
    hipLaunchKernelGGL(combine_bwd_kernel<BF16>, grid, dim3(256), 0, s, gg, yy, row_map, topk_w,
                       T, k, T * k, chunks, dd, d_topk_w);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<F32>, grid, dim3(256), 0, s, gg, yy, row_map, topk_w,
                       T, k, T * k, chunks, dd, d_topk_w);
  return launch_status();
}

moe_status_t moe_repack_glu_weights(const void* w, const float* b, int dtype, int E, int f,
                                    int d, int inverse, void* w_out, float* b_out,
                                    void* stream) {
  const int G = moe_glu_granularity();
  MOE_CHECK_ARG(E >= 1 && f > 0 && d > 0 && valid_dtype(dtype) && f % G == 0);
  MOE_CHECK_ARG(w && w_out && w != w_out && aligned16(w) && aligned16(w_out));
  MOE_CHECK_ARG((b == nullptr) == (b_out == nullptr));
  MOE_CHECK_ARG(b == nullptr || (const void*)b != (const void*)b_out);
  MOE_CHECK_ARG((d * dtype_size(dtype)) % 16 == 0);
  int chunks = (int)(d * dtype_size(dtype) / 16);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  size_t rows = (size_t)E * 2 * f;
  MOE_CHECK_ARG(rows < (size_t)INT32_MAX);
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(w), b, E, f, G, chunks, inverse,
                     reinterpret_cast<u32x4*>(w_out), b_out);
  return launch_status();
}

}  // extern "C"
