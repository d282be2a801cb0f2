// Top-k routing and its backward.
//
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上", section
// "MoE ブロックにおけるトレーニングのボトルネック克服": the tokens each expert
// receives are a run-time quantity; computing them on the host stalls the GPU.
// Here selection, gates and (in the permute) the counts stay on the device.
//
// One thread per token keeps a sorted list of the best k (logit, id) pairs in
// registers (static indexing, so the list never spills): a candidate walks the
// list and swaps with every entry it beats.  Strictly-greater comparison keeps
// the lower id first among equal logits.  The logits row is only E floats, so
// the kernel is latency-bound and tiny next to the GEMMs.
#include "common.hpp"
#include "route.hpp"

#include <math.h>

namespace moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int MAXK>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int score, int normalize,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ w,
                                                         int32_t* err_word) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  route_select<MAXK>(logits + (size_t)t * E, E, k, score, normalize, idx + (size_t)t * k,
                     w + (size_t)t * k, err_word);
}

template <int MAXK>
__global__ void __launch_bounds__(256) route_topk_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, int T, int E, int k, int score, int normalize,
    float* __restrict__ dl) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float* out = dl + (size_t)t * E;
  int ii[MAXK];
  float lv[MAXK], gv[MAXK], dv[MAXK];
  float S = 0.0f;
#pragma unroll
  for (int p = 0; p < MAXK; ++p)
    if (p < k) {
      int e = idx[(size_t)t * k + p];
      e = (e < 0 || e >= E) ? 0 : e;
      ii[p] = e;
      float v = row[e];
      lv[p] = (v == v) ? v : -INFINITY;
      dv[p] = dw[(size_t)t * k + p];
    }
  if (score == MOE_SCORE_SOFTMAX && !normalize) {
    // p_m = softmax over all E;  dl_m = p_m (g_m - sum_j p_j g_j), g = dw scattered
    float mall = -INFINITY;
    for (int e = 0; e < E; ++e) {
      float v = row[e];
      if (v == v) mall = fmaxf(mall, v);
    }
    float Z = 0.0f;
    for (int e = 0; e < E; ++e) {
      float v = row[e];
      if (v == v) Z += expf(v - mall);
    }
    float inner = 0.0f;
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) inner += expf(lv[p] - mall) / Z * dv[p];
    for (int e = 0; e < E; ++e) {
      float v = row[e];
      float pe = (v == v) ? expf(v - mall) / Z : 0.0f;
      float ge = 0.0f;
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k && ii[p] == e) ge += dv[p];
      out[e] = pe * (ge - inner);
    }
    return;
  }
  for (int e = 0; e < E; ++e) out[e] = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    float m = lv[0];
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) m = fmaxf(m, lv[p]);
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) {
        gv[p] = expf(lv[p] - m);
        S += gv[p];
      }
    float inner = 0.0f;
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) inner += gv[p] / S * dv[p];
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) out[ii[p]] = gv[p] / S * (dv[p] - inner);
  } else {
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) {
        gv[p] = route_sigmoid(lv[p]);
        S += gv[p];
      }
    if (normalize) {
      float inner = 0.0f;
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k) inner += gv[p] / S * dv[p];
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k) out[ii[p]] = gv[p] * (1.0f - gv[p]) / S * (dv[p] - inner);
    } else {
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k) out[ii[p]] = dv[p] * gv[p] * (1.0f - gv[p]);
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status_t moe_route_topk(const float* logits, int T, int E, int k, int score, int normalize,
                            int32_t* topk_idx, float* topk_w, int32_t* err_word, void* stream) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= E &&
                k <= MOE_MAX_TOPK);
  MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(logits && topk_idx && topk_w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((T + 255) / 256), block(256);
  if (k <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, score,
                       normalize, topk_idx, topk_w, err_word);
  else
    hipLaunchKernelGGL(route_topk_kernel<MOE_MAX_TOPK>, grid, block, 0, s, logits, T, E, k,
                       score, normalize, topk_idx, topk_w, err_word);
  return launch_status();
}

moe_status_t moe_route_topk_bwd(const float* logits, const int32_t* topk_idx,
                                const float* d_topk_w, int T, int E, int k, int score,
                                int normalize, float* d_logits, void* stream) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= E &&
                k <= MOE_MAX_TOPK);
  MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(logits && topk_idx && d_topk_w && d_logits);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((T + 255) / 256), block(256);
  if (k <= 8)
    hipLaunchKernelGGL(route_topk_bwd_kernel<8>, grid, block, 0, s, logits, topk_idx, d_topk_w,
                       T, E, k, score, normalize, d_logits);
  else
    hipLaunchKernelGGL(route_topk_bwd_kernel<MOE_MAX_TOPK>, grid, block, 0, s, logits,
                       topk_idx, d_topk_w, T, E, k, score, normalize, d_logits);
  return launch_status();
}

}  // extern "C"
