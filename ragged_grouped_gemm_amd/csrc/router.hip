// The router's linear map fused with top-k routing, and its backward.
//
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上":
//  - "MoE ブロックにおけるトレーニングのボトルネック克服": the tokens each expert
//    receives come out of routing at run time (and are usually handled on the
//    CPU); here they never leave the GPU;
//  - Figure 1: the forward and the backward pass fused into custom kernels.
// The router itself (logits = x Wr^T, no bias) is the plain reading of the
// layer's input to its routing; the pages do not write it out.
//
// Forward, one launch (moe_router_topk): a workgroup takes 32 tokens; its 8
// waves split the reduction over d, each accumulating a 32 x 32 block of
// logits per 32-expert tile with v_mfma_f32_32x32x16_bf16 from operands read
// straight from memory (x rows once, the router weights from L2); the waves'
// partial sums are added in wave order through LDS, the logits are written
// out (the backward needs them) and selected in LDS with the same
// selection and gate code as moe_route_topk.  Up to RT_MAXE experts per pass;
// more experts compute the logits in passes and select with moe_route_topk's
// kernel.
//
// Backward (moe_router_bwd): dWr = dlogits^T x on float32 MFMA (a workgroup
// owns 32 columns of d and 32 experts, its waves split the tokens and their
// tiles are added in wave order) and dx += dlogits Wr (a thread 8 columns of
// 8 tokens, experts in order, one rounding).
// Both are deterministic; there are no atomics.
#include "common.hpp"
#include "route.hpp"

namespace moe {

static constexpr int RT_TOK = 32;     // tokens per workgroup
static constexpr int RT_WAVES = 8;    // waves per workgroup, splitting d
static constexpr int RT_MAXE = 256;   // experts per pass (selection kept in LDS)

// acc[4 g + q] += sum over the step's 16 k of x[token r][k] Wr[expert 8 g + 4 h + q][k],
// r = lane & 31, h = lane >> 5 (the router weights are the MFMA's first operand).
__device__ __forceinline__ void rmma(f32x16& acc, const u32x4& wv, const u32x4& xv) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv),
                                                __builtin_bit_cast(bf16x8, xv), acc, 0, 0, 0);
}

// NT 32-expert tiles (experts e0 .. e0 + ne - 1 of E, ne <= 32 NT), U k-steps of
// loads in flight.  Logits row stride E; select: also route (ne == E).
template <int NT, int U, int MAXK>
__global__ void __launch_bounds__(RT_WAVES * 64)
    router_topk_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T,
                       int d, int E, int e0, int ne, int k, int score, int normalize,
                       float* __restrict__ logits, int32_t* __restrict__ idx,
                       float* __restrict__ w, int32_t* err_word, int select) {
  extern __shared__ float rt_smem[];
  float* part = rt_smem;                           // [RT_WAVES][32][33]
  float* lg = rt_smem + RT_WAVES * 32 * 33;        // [32][NT * 32 + 1]
  constexpr int LGS = NT * 32 + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TOK;
  const int r = lane & 31, h = lane >> 5;
  // rows past T or experts past ne read valid rows; their results are dropped
  const int tok = min(t0 + r, T - 1);
  const int nsteps = d / 16;
  const int s0 = wave * nsteps / RT_WAVES, s1 = (wave + 1) * nsteps / RT_WAVES;
  // the lane's 16 bytes of step s: k = 16 s + 8 h .. + 7 = 16-byte chunk 2 s + h of the row
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)tok * d) + h;
  const u32x4* wrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int e = e0 + min(32 * j + r, ne - 1);
    wrow[j] = reinterpret_cast<const u32x4*>(wr + (size_t)e * d) + h;
  }
  f32x16 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  int s = s0;
  for (; s + U <= s1; s += U) {
    u32x4 xa[U], wb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xa[u] = xr[2 * (s + u)];
#pragma unroll
      for (int j = 0; j < NT; ++j) wb[u][j] = wrow[j][2 * (s + u)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) rmma(acc[j], wb[u][j], xa[u]);
  }
  for (; s < s1; ++s) {
    const u32x4 xa = xr[2 * s];
#pragma unroll
    for (int j = 0; j < NT; ++j) rmma(acc[j], wrow[j][2 * s], xa);
  }
  // the waves' partial sums, added in wave order (wave i covers the i-th
  // slice of d), one 32-expert tile at a time
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    float* pw = part + wave * 32 * 33 + r * 33;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) pw[8 * g + 4 * h + q] = acc[j][4 * g + q];
    __syncthreads();
    for (int i = tid; i < 32 * 32; i += RT_WAVES * 64) {
      const int rr = i >> 5, cc = i & 31;
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < RT_WAVES; ++wv) v += part[wv * 32 * 33 + rr * 33 + cc];
      lg[rr * LGS + 32 * j + cc] = v;
    }
    __syncthreads();
  }
  if (logits) {
    for (int i = tid; i < RT_TOK * ne; i += RT_WAVES * 64) {
      const int rr = i / ne, e = i - rr * ne;
      if (t0 + rr < T) logits[(size_t)(t0 + rr) * E + e0 + e] = lg[rr * LGS + e];
    }
  }
  if (select && tid < RT_TOK && t0 + tid < T)
    route_select<MAXK>(lg + tid * LGS, ne, k, score, normalize, idx + (size_t)(t0 + tid) * k,
                       w + (size_t)(t0 + tid) * k, err_word);
}

template <int NT, int U, int MAXK>
moe_status_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int e0,
                           int ne, int k, int score, int normalize, float* logits, int32_t* idx,
                           float* w, int32_t* err, int select, hipStream_t s) {
  auto kern = router_topk_kernel<NT, U, MAXK>;
  const size_t lds = (size_t)(RT_WAVES * 32 * 33 + RT_TOK * (NT * 32 + 1)) * sizeof(float);
  static bool attr_set[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  if (!attr_set[dev]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return MOE_ERR_HIP;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(kern, dim3((T + RT_TOK - 1) / RT_TOK), dim3(RT_WAVES * 64), lds, s, x, wr,
                     T, d, E, e0, ne, k, score, normalize, logits, idx, w, err, select);
  return launch_status();
}

// One pass over experts e0 .. e0 + ne - 1 (ne <= RT_MAXE).
template <int MAXK>
moe_status_t router_pass(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int e0,
                         int ne, int k, int score, int normalize, float* logits, int32_t* idx,
                         float* w, int32_t* err, int select, hipStream_t s) {
  if (ne <= 32)
    return launch_router<1, 4, MAXK>(x, wr, T, d, E, e0, ne, k, score, normalize, logits, idx, w,
                                     err, select, s);
  if (ne <= 64)
    return launch_router<2, 4, MAXK>(x, wr, T, d, E, e0, ne, k, score, normalize, logits, idx, w,
                                     err, select, s);
  if (ne <= 128)
    return launch_router<4, 2, MAXK>(x, wr, T, d, E, e0, ne, k, score, normalize, logits, idx, w,
                                     err, select, s);
  return launch_router<8, 2, MAXK>(x, wr, T, d, E, e0, ne, k, score, normalize, logits, idx, w,
                                   err, select, s);
}

// dWr[e][c] (+)= sum over t of dl[t][e] x[t][c] for the 32 experts e0 ..
// e0 + 31 (fewer at the end) and the 32 columns c0 .. c0 + 31 of one
// workgroup: the contraction over tokens on v_mfma_f32_32x32x2f32 (float32
// products and sums; bf16 x is exact in float32).  Per MFMA, lane l holds
// dl[t + (l >> 5)][e0 + (l & 31)] (first operand: row = expert, k = token)
// and x[t + (l >> 5)][c0 + (l & 31)] (second: k = token, column); the result
// register 4 g + q of lane l is expert 8 g + 4 (l >> 5) + q, column l & 31.
// Wave w takes the token pairs of the blocks w, w + RB_WAVES, ... of RB_PAIRS
// pairs, loading the next block while multiplying the current one; the
// waves' tiles are added in wave order through LDS.  Column tiles are spread
// so that neighbouring tiles (which share 128-byte lines of x) run on one
// XCD.
static constexpr int RB_WAVES = 8;
static constexpr int RB_PAIRS = 16;

__global__ void __launch_bounds__(RB_WAVES * 64) router_dwr_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dl, int T, int d, int E,
    float* __restrict__ dwr, int accumulate) {
  __shared__ float part[RB_WAVES][32][33];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b % 8, q8 = nb / 8, r8 = nb % 8;
  const int c0 = (xcd * q8 + min(xcd, r8) + b / 8) * 32;
  const int e0 = blockIdx.y * 32;
  const int h = lane >> 5, el = e0 + (lane & 31);
  const bool ev = el < E;
  const int npairs = (T + 1) / 2;
  // x is kept as its bf16 bits until the MFMA that uses it (a conversion
  // right after the load would wait for it there)
  float a[2][RB_PAIRS];
  uint32_t bx[2][RB_PAIRS];
  // buffer loads over the rows from the block's first token on: rows past T
  // (and experts past E) read as zero, so every block is loaded without a
  // branch (a block wholly past T has an empty range and touches nothing)
  auto records = [](long long b) { return (int)(b < 0 ? 0 : b > 0x7ffffff0LL ? 0x7ffffff0LL : b); };
  auto load = [&](int buf, int p0) {
    const long long tb = 2LL * p0;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x) + (tb < T ? tb * d + c0 : 0), (short)0,
        records(((T - tb) * d - c0) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(dl) + (tb < T ? tb * E : 0), (short)0, records((T - tb) * E * 4),
        0x00020000);
#pragma unroll
    for (int i = 0; i < RB_PAIRS; ++i) {
      const int r = 2 * i + h;
      const uint32_t go = ev ? (uint32_t)(r * E + el) * 4u : 0x80000000u;
      a[buf][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, go, 0, 0));
      bx[buf][i] = __builtin_amdgcn_raw_buffer_load_b16(xr, (uint32_t)(r * d + (lane & 31)) * 2u,
                                                        0, 0);
    }
  };
  f32x16 acc = {};
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RB_PAIRS; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[buf][i],
                                                 __builtin_bit_cast(float, bx[buf][i] << 16),
                                                 acc, 0, 0, 0);
  };
  // the next block's loads are issued before this block's MFMAs (the
  // scheduling barriers keep them there); blocks go in pairs, a block past
  // the tokens adding exact zeros, so that no branch stands between a load
  // and its use
  constexpr int STRIDE = RB_WAVES * RB_PAIRS;
  int p0 = wave * RB_PAIRS;
  const int nblk = p0 < npairs ? (npairs - p0 + STRIDE - 1) / STRIDE : 0;
  load(0, p0);
  for (int j = 0; j < (nblk + 1) / 2; ++j, p0 += 2 * STRIDE) {
    load(1, p0 + STRIDE);
    __builtin_amdgcn_sched_barrier(0);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    load(0, p0 + 2 * STRIDE);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) part[wave][8 * (r >> 2) + 4 * h + (r & 3)][lane & 31] = acc[r];
  __syncthreads();
  for (int i = tid; i < 32 * 32; i += RB_WAVES * 64) {
    const int e = i >> 5, c = i & 31;
    if (e0 + e >= E) break;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < RB_WAVES; ++w) v += part[w][e][c];
    float* o = dwr + (size_t)(e0 + e) * d + c0 + c;
    *o = accumulate ? *o + v : v;
  }
}

// dx[t][c .. c + 7] = bf16(dx + sum over e of dl[t][e] Wr[e][c .. c + 7]) for
// RD_TOK tokens t of the workgroup row blockIdx.y (their expert gradients are
// the same for the whole workgroup): each thread 8 columns, each 16-byte
// chunk of the router weights used for all RD_TOK tokens.
static constexpr int RD_TOK = 8;
static constexpr int RD_THREADS = 128;

__global__ void __launch_bounds__(RD_THREADS) router_dx_kernel(const float* __restrict__ dl,
                                                               const uint16_t* __restrict__ wr,
                                                               int T, int d, int E,
                                                               uint16_t* __restrict__ dx) {
  const int t0 = blockIdx.y * RD_TOK;
  const int c = (blockIdx.x * RD_THREADS + threadIdx.x) * 8;
  if (c >= d) return;
  const int nt = min(RD_TOK, T - t0);
  float acc[RD_TOK][8];
#pragma unroll
  for (int j = 0; j < RD_TOK; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[j][q] = 0.0f;
  const float* g = dl + (size_t)t0 * E;
  // rows past the last token re-read its gradients: their sums are never
  // stored
  auto fma_chunk = [&](const u32x4& raw, int e) {
    float v[8];
    unpack_chunk(raw, v, BF16());
#pragma unroll
    for (int j = 0; j < RD_TOK; ++j) {
      const float ge = g[(size_t)min(j, nt - 1) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[j][q] += ge * v[q];
    }
  };
  // experts in groups of 8 (their chunks loaded together), then one by one
  constexpr int EU = 8;
  int e = 0;
  for (; e + EU <= E; e += EU) {
    u32x4 raw[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u)
      raw[u] = *reinterpret_cast<const u32x4*>(wr + (size_t)(e + u) * d + c);
#pragma unroll
    for (int u = 0; u < EU; ++u) fma_chunk(raw[u], e + u);
  }
  for (; e < E; ++e) fma_chunk(*reinterpret_cast<const u32x4*>(wr + (size_t)e * d + c), e);
#pragma unroll
  for (int j = 0; j < RD_TOK; ++j) {
    if (j >= nt) break;
    u32x4* p = reinterpret_cast<u32x4*>(dx + (size_t)(t0 + j) * d + c);
    float v[8];
    unpack_chunk(*p, v, BF16());
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += acc[j][q];
    *p = pack_chunk(v, BF16());
  }
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_router_topk(const void* x, const void* w_router, int dtype, int T, int d, int E,
                             int k, int score, int normalize, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* err_word, void* stream) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= E &&
                k <= MOE_MAX_TOPK && d > 0 && d % 32 == 0);
  MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID);
  if (dtype != MOE_BF16) return valid_dtype(dtype) ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  MOE_CHECK_ARG((topk_idx == nullptr) == (topk_w == nullptr));
  MOE_CHECK_ARG(topk_idx || logits);
  MOE_CHECK_ARG(E <= RT_MAXE || logits);         // more experts select from the written logits
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_router && aligned16(x) && aligned16(w_router));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w_router);
  const bool select = topk_idx != nullptr;
  if (E <= RT_MAXE) {
    if (k <= 8)
      return router_pass<8>(xb, wb, T, d, E, 0, E, k, score, normalize, logits, topk_idx, topk_w,
                            err_word, select, s);
    return router_pass<MOE_MAX_TOPK>(xb, wb, T, d, E, 0, E, k, score, normalize, logits,
                                     topk_idx, topk_w, err_word, select, s);
  }
  for (int e0 = 0; e0 < E; e0 += RT_MAXE) {
    moe_status_t st = router_pass<8>(xb, wb, T, d, E, e0, E - e0 < RT_MAXE ? E - e0 : RT_MAXE, k,
                                     score, normalize, logits, nullptr, nullptr, nullptr, 0, s);
    if (st != MOE_OK) return st;
  }
  return select ? moe_route_topk(logits, T, E, k, score, normalize, topk_idx, topk_w, err_word,
                                 stream)
                : MOE_OK;
}

moe_status_t moe_router_bwd(const void* x, const void* w_router, int dtype, const float* d_logits,
                            int T, int d, int E, float* d_w_router, int accumulate, void* dx,
                            void* stream) {
  // d bounded so that 32 rows of x stay within a buffer load's 32-bit offsets
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && d > 0 && d % 32 == 0 &&
                d <= (1 << 20));
  if (dtype != MOE_BF16) return valid_dtype(dtype) ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d_w_router && T > 0) {
    MOE_CHECK_ARG(x && d_logits && aligned16(x));
    hipLaunchKernelGGL(router_dwr_kernel, dim3(d / 32, (E + 31) / 32),
                       dim3(RB_WAVES * 64), 0, s, static_cast<const uint16_t*>(x), d_logits, T,
                       d, E, d_w_router, accumulate);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  if (dx && T > 0) {
    MOE_CHECK_ARG(w_router && d_logits && aligned16(w_router) && aligned16(dx));
    hipLaunchKernelGGL(router_dx_kernel,
                       dim3((d / 8 + RD_THREADS - 1) / RD_THREADS, (T + RD_TOK - 1) / RD_TOK),
                       dim3(RD_THREADS), 0, s,
                       d_logits, static_cast<const uint16_t*>(w_router), T, d, E,
                       static_cast<uint16_t*>(dx));
    return launch_status();
  }
  return MOE_OK;
}

}  // extern "C"
