// Top-k selection and gate weights of one token's router logits, shared by
// the routing kernel (logits from memory) and the fused router (logits in LDS),
// so both select and weigh bit-identically.
//
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上", section "MoE ブロック
// におけるトレーニングのボトルネック克服": the tokens per expert come out of
// routing at run time.  The pages give no gate formula; the reading taken:
// the k largest logits (equal logits: the lower expert id first, NaN ranked
// as -inf and reported), gates softmax over the selection (= the full softmax
// renormalised) or sigmoid / sum over the selection, `normalize` = 0 keeping
// the unrenormalised probabilities.
#pragma once

#include "common.hpp"

#include <math.h>

namespace moe {

__device__ __forceinline__ float route_sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// row: E logits of one token (global or LDS); writes idx[0..k), w[0..k).
template <int MAXK>
__device__ __forceinline__ void route_select(const float* row, int E, int k, int score,
                                             int normalize, int32_t* idx, float* w,
                                             int32_t* err_word) {
  float bv[MAXK];
  int bi[MAXK];
#pragma unroll
  for (int p = 0; p < MAXK; ++p) {
    bv[p] = -INFINITY;
    bi[p] = -1;
  }
  bool nan_seen = false;
  for (int e = 0; e < E; ++e) {
    float v = row[e];
    if (v != v) {
      nan_seen = true;
      v = -INFINITY;
    }
    int id = e;
#pragma unroll
    for (int p = 0; p < MAXK; ++p) {
      // (v, id) beats the entry when its logit is larger, or equal with a lower
      // id (a displaced entry carried down the list may tie a later entry)
      bool take = (p < k) && (bi[p] < 0 || v > bv[p] || (v == bv[p] && id >= 0 && id < bi[p]));
      float tv = bv[p];
      int ti = bi[p];
      bv[p] = take ? v : tv;
      bi[p] = take ? id : ti;
      v = take ? tv : v;
      id = take ? ti : id;
    }
  }
  if (nan_seen) set_err(err_word, MOE_ERRBIT_NAN_LOGIT);

  float g[MAXK];
  float s = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    float m = bv[0];
    if (normalize) {
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k) {
          g[p] = expf(bv[p] - m);
          s += g[p];
        }
    } else {
      float mall = -INFINITY;
      for (int e = 0; e < E; ++e) {
        float v = row[e];
        if (v == v) mall = fmaxf(mall, v);
      }
      for (int e = 0; e < E; ++e) {
        float v = row[e];
        if (v == v) s += expf(v - mall);
      }
#pragma unroll
      for (int p = 0; p < MAXK; ++p)
        if (p < k) g[p] = expf(bv[p] - mall);
    }
  } else {
#pragma unroll
    for (int p = 0; p < MAXK; ++p)
      if (p < k) {
        g[p] = route_sigmoid(bv[p]);
        s += g[p];
      }
    if (!normalize) s = 1.0f;
  }
#pragma unroll
  for (int p = 0; p < MAXK; ++p)
    if (p < k) {
      idx[p] = bi[p];
      w[p] = (score == MOE_SCORE_SOFTMAX || normalize) ? g[p] / s : g[p];
    }
}

}  // namespace moe
