/*
 * moe.h — C ABI of the MI355X (gfx950) dropless MoE expert-FFN library.
 *
 * The layer, for T tokens of width d routed to k of E local experts (R = T*k
 * routed rows), each expert an FFN of width f:
 *
 *   route top-k  ->  permute into expert-contiguous rows  ->  FC1 grouped GEMM
 *   with a fused GLU epilogue  ->  FC2 grouped GEMM  ->  weighted combine,
 *
 * and the backward pass (combine backward, FC2 dgrad with a fused dGLU
 * epilogue, weight gradients, FC1 dgrad, unpermute-sum, route backward).
 *
 * Sources (page title and section):
 *  [P1] "高度な融合カーネルによる MoE 学習スループットの向上" (NVIDIA developer-blog
 *       post on fused MoE kernels, Japanese rendering):
 *       - "MoE ブロックにおけるトレーニングのボトルネック克服": per-expert token
 *         counts are a run-time quantity; kernel families GroupGemm + Quantize,
 *         GroupGemm + Activation, GroupGemm + dActivation; SwiGLU, GeGLU and
 *         sReLU with clamp and scaling options.
 *       - "融合された GEMM エピローグによる GLU 活性化関数の最適化" (+ Figure 2):
 *         GLU epilogue on weights repacked into interleaved input/gate column
 *         tiles; dSwiGLU in the backward epilogue; feature scaling, clamp and
 *         bias-vector add in the epilogue.
 *       - "ホストとデバイスの同期および CPU 起動オーバーヘッドの排除": the grouped
 *         GEMM reads the tokens per group from GPU memory, so no host sync is
 *         needed and the whole iteration can be graph-captured.
 *       - "カーネルレベルでの向上から事前学習全体の速度向上へ": dynamic
 *         scheduling and a configurable limit on the compute units a kernel uses.
 *  [P2] "JAXとNVIDIA Transformer EngineによるDropless MoE学習の高速化",
 *       section "主張と根拠": dropless MoE over ragged tensors, one grouped GEMM
 *       call over all ragged groups; tokens are dispatched to the experts and
 *       their results combined.
 *  [P3] "FlashMoE: Fast Distributed MoE in a Single Kernel", Abstract: a MoE
 *       operator as dispatch, expert compute and combine phases.
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees, copies device->host or synchronises.  Each call
 *    only enqueues kernels on `stream` (a hipStream_t; NULL = default stream),
 *    so every call may be recorded into a HIP graph.
 *  - Tensors are dense and row-major.  Sizes known on the host (T, d, f, E, k)
 *    are ints; the routing-dependent sizes (per-expert counts and offsets)
 *    exist only in device memory and are read there by the kernels.
 *  - Weights use the [out, in] convention: W1 [E, n1, d] (n1 = 2f for gated
 *    activations, f for squared ReLU), W2 [E, d, f].  Biases are float32.
 *  - Element types: MOE_F32 (float32) or MOE_BF16 (bfloat16, round to nearest
 *    even on store, float32 accumulation).
 *  - Alignment: every pointer 16-byte aligned; d and f multiples of 32.
 *  - Errors: argument errors are returned synchronously as a status code and
 *    nothing is enqueued.  A failed kernel launch returns MOE_ERR_HIP.  Data
 *    errors found on the device (NaN logits, expert ids out of range) never
 *    stop the kernels; they OR bits into the optional device word `err_word`
 *    (MOE_ERRBIT_*), which the caller may read at any time.
 *  - Results are deterministic: no floating-point atomics anywhere.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, k > E ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented combination */
  MOE_ERR_WORKSPACE = 3,    /* workspace too small */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_E4M3 = 2, /* MXFP8 GEMM operands (moe_mx_t); see the MXFP8 section below */
  MOE_E2M1 = 3  /* MXFP4 GEMM operands (moe_mx_t, two codes per byte), same section */
} moe_dtype_t;

/* An MXFP8 or MXFP4 matrix (layout and format in the MXFP8 section below). */
typedef struct {
  uint8_t* data;   /* E4M3 codes [rows, ld] or E2M1 codes [rows, ld / 2] bytes */
  uint8_t* scale;  /* E8M0 codes [rows, ld / 32] */
  int64_t ld;      /* elements per row, a multiple of 32 */
} moe_mx_t;


typedef enum {
  MOE_ACT_SWIGLU = 0,  /* silu_a(gate) * lin,  silu_a(g) = g * sigmoid(a g)   */
  MOE_ACT_GEGLU = 1,   /* gelu(gate) * lin (erf form; tanh form by flag)        */
  MOE_ACT_SRELU = 2    /* relu(h)^2, not gated: FC1 has n1 = f output columns   */
} moe_act_t;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_t;

typedef enum { MOE_BWD_DGRAD = 0, MOE_BWD_WGRAD = 1 } moe_bwd_mode_t;

#define MOE_ERRBIT_NAN_LOGIT 1u    /* a router logit was NaN (ranked as -inf)   */
#define MOE_ERRBIT_BAD_EXPERT 2u   /* an expert id outside [0, E) (counted as 0) */

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* Library version string and readable status names. */
const char* moe_version(void);
const char* moe_status_string(moe_status_t s);

/* Rows per repack chunk G of the packed FC1 weight layout (see
 * moe_repack_glu_weights).  f must be a multiple of G. */
int moe_glu_granularity(void);

/* ---------------------------------------------------------------- routing
 * a1.  Top-k routing [P1 "MoE ブロックにおけるトレーニングのボトルネック克服"].
 *   logits   [T, E] float32 (in)
 *   topk_idx [T, k] int32 (out): the k experts with the largest logits,
 *            largest first; equal logits are taken in increasing expert id;
 *            NaN logits rank as -inf and set MOE_ERRBIT_NAN_LOGIT.
 *   topk_w   [T, k] float32 (out): gate weights.  SOFTMAX: softmax over the
 *            selected logits when `normalize` (= full softmax renormalised
 *            over the selection), else the full-softmax probabilities.
 *            SIGMOID: sigmoid(l) / sum over the selection when `normalize`,
 *            else sigmoid(l).
 *   err_word int32 device word (in/out, nullable).
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS. */
moe_status_t moe_route_topk(const float* logits, int T, int E, int k, int score, int normalize,
                            int32_t* topk_idx, float* topk_w, int32_t* err_word, void* stream);

/* a7.  Gradient of the gate weights with respect to the logits.  The pages
 * name the router only as part of the MoE block [P1 "MoE ブロックにおける
 * トレーニングのボトルネック克服"] and give no gate formula; the gate
 * functions are the reading stated at moe_route_topk (softmax over the
 * selection, or sigmoid normalised over it), and this is their exact
 * Jacobian-vector product: the selection itself is piecewise constant.
 *   softmax, normalised:  dl_j = w_j (dw_j - sum_i w_i dw_i) for selected j;
 *   sigmoid, normalised:  dl_j = s_j (1 - s_j) / S (dw_j - sum_i w_i dw_i),
 *                         s = sigmoid(l), S = sum over the selection.
 *   logits   [T, E] float32 (in, the forward's logits); topk_idx [T, k] (in)
 *   d_topk_w [T, k] float32 (in): dLoss/dtopk_w;  d_logits [T, E] float32
 *   (out, fully overwritten; 0 for unselected experts except for the
 *   unnormalised softmax, whose denominator involves every logit).
 * Argument errors (null pointers, k out of range) return a status code. */
moe_status_t moe_route_topk_bwd(const float* logits, const int32_t* topk_idx,
                                const float* d_topk_w, int T, int E, int k, int score,
                                int normalize, float* d_logits, void* stream);

/* f4.  The router's linear map fused with top-k routing [P1 "MoE ブロックにおける
 * トレーニングのボトルネック克服": the tokens per expert come out of routing at
 * run time; P1 Figure 1: forward and backward fused into custom kernels].  The
 * pages do not write the router out; the reading taken is a linear map of the
 * layer's input without bias:
 *   logits[t, e] = sum_c x[t, c] w_router[e, c]      (float32 accumulation)
 * followed, in the same launch and from the logits held in LDS, by exactly
 * the selection and gates of moe_route_topk (bit-identical to moe_route_topk
 * on the same logits).
 *   x [T, d], w_router [E, d]: dtype MOE_BF16 (MOE_F32: MOE_ERR_UNSUPPORTED),
 *   d a multiple of 32, 16-byte aligned pointers.
 *   logits   [T, E] float32 (out, nullable for E <= 256; the routing backward
 *            needs it).  For E > 256 the logits are computed in passes of 256
 *            experts and selected by moe_route_topk's kernel: logits required.
 *   topk_idx [T, k], topk_w [T, k] (out, as moe_route_topk; both NULL: only
 *            the logits are computed); err_word as moe_route_topk.
 * Argument errors return a status code before anything is enqueued. */
moe_status_t moe_router_topk(const void* x, const void* w_router, int dtype, int T, int d, int E,
                             int k, int score, int normalize, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* err_word, void* stream);

/* Backward of the router's map (same reading), given d_logits [T, E] float32
 * (moe_route_topk_bwd's output):
 *   d_w_router [E, d] float32 (out, nullable): sum over tokens of
 *              d_logits[t, e] x[t], summed in token order (added to the
 *              existing values when `accumulate`);
 *   dx         [T, d] bf16 (in/out, nullable): dx[t] += sum_e d_logits[t, e]
 *              w_router[e], the router's share of the layer's input gradient,
 *              summed in float32 over experts in order and rounded once.
 * x, w_router as moe_router_topk; d at most 2^20.  Both sums are taken in a
 * fixed order (no atomics): the same inputs give the same bits. */
moe_status_t moe_router_bwd(const void* x, const void* w_router, int dtype, const float* d_logits,
                            int T, int d, int E, float* d_w_router, int accumulate, void* dx,
                            void* stream);

/* ---------------------------------------------------------------- permute
 * a2.  Expert-contiguous layout [P2 "主張と根拠"; P1 "ホストとデバイスの同期…"].
 * The row of assignment i = t*k + j (expert e) is
 *     offsets[e] + #{ i' < i : expert(i') = e }
 * (a stable counting sort by expert).
 *   x          [T, d] dtype (in); may be NULL when xp is NULL.
 *   topk_idx   [T, k] int32 (in)
 *   counts     [E] int32 (out), offsets [E+1] int32 (out, exclusive scan,
 *              offsets[E] = T*k), pad_offsets [E+1] int32 (out, nullable:
 *              offsets of the segments padded to multiples of 32 rows)
 *   row_map    [T, k] int32 (out): row of each assignment
 *   src_row    [T*k] int32 (out): token of each row
 *   xp         [T*k, d] dtype (out, nullable): xp[r] = x[src_row[r]]
 *   ws         device workspace of at least moe_permute_workspace_size() bytes
 * Ids outside [0, E) set MOE_ERRBIT_BAD_EXPERT and are counted as expert 0,
 * so the outputs always form a valid permutation. */
size_t moe_permute_workspace_size(int T, int E, int k);
moe_status_t moe_permute(const void* x, int dtype, int T, int d, const int32_t* topk_idx,
                         int k, int E, int32_t* counts, int32_t* offsets,
                         int32_t* pad_offsets, int32_t* row_map, int32_t* src_row, void* xp,
                         void* ws, size_t ws_bytes, int32_t* err_word, void* stream);

/* a2 without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Computes exactly what moe_permute computes, with the same
 * arguments except ws / ws_bytes: the per-chunk counts live in a static
 * device array of MOE_PERMUTE_NOALLOC_MAX_BYTES bytes inside the library,
 * one per GPU, held until the process ends.  The call allocates and frees
 * nothing; its first call on a device looks up that device's copy of the
 * array (make one call before capturing a graph).
 *   Limit: moe_permute_workspace_size(T, E, k) <= MOE_PERMUTE_NOALLOC_MAX_BYTES,
 *   i.e. ceil(T*k / 1024) * E <= 262144 (for example T*k <= 8M at E = 32,
 *   T*k <= 256K at E = 1024); larger sizes return MOE_ERR_WORKSPACE before
 *   anything is enqueued.
 *   Every call on one GPU uses the same array (nothing in it needs clearing:
 *   each call writes every entry before reading it), so calls that overlap on
 *   one GPU -- on different streams, or from different host threads without
 *   ordering -- race and must not be made. */
#define MOE_PERMUTE_NOALLOC_MAX_BYTES (1 << 20)
moe_status_t moe_permute_noalloc(const void* x, int dtype, int T, int d,
                                 const int32_t* topk_idx, int k, int E, int32_t* counts,
                                 int32_t* offsets, int32_t* pad_offsets, int32_t* row_map,
                                 int32_t* src_row, void* xp, int32_t* err_word, void* stream);

/* ---------------------------------------------------------------- repack
 * a13.  FC1 weight repack [P1 "融合された GEMM エピローグ…", Figure 2].
 * Canonical W1 rows [0, f) are the gate chunk (activated) and [f, 2f) the
 * linear chunk.  The packed layout alternates G-row chunks (G =
 * moe_glu_granularity()): gate chunk c -> packed rows [2Gc, 2Gc+G), linear
 * chunk c -> [2Gc+G, 2Gc+2G), so every 2G-wide output tile of FC1 holds the
 * matching gate and linear columns.  A bit-exact row permutation.
 *   w   [E, 2f, d] dtype (in), b [E, 2f] float32 (in, nullable)
 *   w_out, b_out: same shapes (out; b_out nullable iff b is); must not alias
 *   inverse = 1 maps packed -> canonical (for exporting dW1 / db1). */
moe_status_t moe_repack_glu_weights(const void* w, const float* b, int dtype, int E, int f,
                                    int d, int inverse, void* w_out, float* b_out,
                                    void* stream);

/* Transposed copy of per-expert weights for the dgrad GEMMs:
 * wt[e][j][i] = w[e][i][j].  The backward products dA = dY W2[e] (FC2) and
 * dXp = dH W1p[e] (FC1) reduce over the rows of the stored weight; with the
 * transposed copy both of their operands are contiguous along the reduction,
 * like the forward GEMMs' (moe_glu_bwd_args_t.w2t, moe_gemm_bwd_args_t.wt).
 * Made once per weight update (the weights do not change within a step).
 *   w  [E, rows, cols] dtype (in), wt [E, cols, rows] dtype (out, must not
 *   alias w); rows and cols multiples of 8; 16-byte aligned pointers.
 * A bit-exact copy; MOE_ERR_INVALID_ARG on bad sizes or pointers. */
moe_status_t moe_transpose_weights(const void* w, int dtype, int E, int rows, int cols, void* wt,
                                   void* stream);

/* A float per assignment moved to the expert-contiguous row order and back
 * (the routing gates as feature-scaling factors of FC1's activation, and
 * their gradients) [P1 "融合された GEMM エピローグ…": feature scaling; P2
 * "主張と根拠": the ragged expert-major layout]:
 *   inverse == 0:  dst[row_map[i]] = src[i]
 *   inverse == 1:  dst[i] = src[row_map[i]]          for i < n = T*k,
 * row_map [T, k] from moe_permute (a permutation of [0, n)); src and dst
 * [n] float32, distinct.  Entries of row_map outside [0, n) are skipped
 * (forward) or give 0 (inverse).  Argument errors return a status code. */
moe_status_t moe_permute_rows(const float* src, const int32_t* row_map, int n, int inverse,
                              float* dst, void* stream);

/* ---------------------------------------------------------------- grouped GEMMs
 * All grouped GEMMs run over the expert segments given by the DEVICE array
 * offsets [E+1] (offsets[0] = 0, nondecreasing, offsets[E] = R); segment e
 * holds rows [offsets[e], offsets[e+1]).  One persistent launch covers every
 * expert: its workgroups read the offsets and enumerate their tiles on the
 * device.  `max_cus` > 0 limits the compute units the launch occupies
 * (0 = all) [P1 "カーネルレベルでの向上…": configurable margin]. */

/* a3.  FC1 with the GLU epilogue [P1 "融合された GEMM エピローグ…"]:
 *   H[r]  = xp[r] @ w1p[e]^T + b1p[e]            (float32 accumulate)
 *   A[r]  = act(gate cols of H, linear cols of H) (see moe_act_t)
 * with optional clamp: gate <- min(gate, L), lin <- clip(lin, -L, L) when
 * clamp > 0 (for SRELU: h <- min(h, L)).
 *   xp  [R, d] dtype;  w1p [E, n1, d] dtype, packed (gated acts);
 *   b1p [E, n1] float32 nullable (packed like w1p);
 *   h_out [R, n1] dtype nullable: pre-activation H saved for the backward;
 *   a_out [R, f] dtype.
 * alpha: slope of SwiGLU's sigmoid (1 = SiLU); gelu_tanh selects GeGLU's
 * tanh form. */
typedef struct {
  size_t struct_size; /* = sizeof(moe_glu_fwd_args_t) */
  int dtype;
  const void* xp;
  const void* w1p;
  const float* b1p;
  const int32_t* offsets;
  int E, R, d, f;
  int act;
  float clamp;
  float alpha;
  int gelu_tanh;
  void* h_out;
  void* a_out;
  int max_cus;
  /* dtype == MOE_E4M3 or MOE_E2M1: xp_mx [R, d] and w1_mx [E*n1, d] (row copies along
   * d) replace xp / w1p; h_out stays bf16; A is written as a_row (row copy
   * [R, f], nullable) and a_col (column copy [f, moe_mx_col_len], nullable,
   * needs pad_offsets), quantized from the float32 epilogue values.  Gated
   * activations only, no bias. */
  const moe_mx_t* xp_mx;
  const moe_mx_t* w1_mx;
  moe_mx_t* a_row;
  moe_mx_t* a_col;
  const int32_t* pad_offsets;
  /* Gather-fused permute (bf16 / float32; nullable, and must be NULL for
   * the MX dtypes, whose row copy is gathered by moe_mx_quantize_experts): with
   * src_row from moe_permute, xp is the unpermuted x [src_rows, d] and row r
   * of the product reads x[src_row[r]], so the permuted copy is never
   * written.  x must span less than 2 GiB; rows whose index lies outside
   * [0, src_rows) read as zeros. */
  const int32_t* src_row;
  int src_rows;
  /* Feature scaling [P1 "融合された GEMM エピローグ…": the epilogues also
   * scale] (nullable, every dtype): row_scale [R] float32, a factor per
   * permuted row multiplying the activation output,
   *   A[r] = row_scale[r] * act(...),
   * applied to the float32 value before A is rounded or quantized.  With the
   * routing gates as factors (moe_permute_rows) the combine then sums with
   * unit weights. */
  const float* row_scale;
} moe_glu_fwd_args_t;
moe_status_t moe_grouped_gemm_glu_fwd(const moe_glu_fwd_args_t* args, void* stream);

/* a4.  Plain grouped GEMM ("linear"): y[r] = a[r] @ w[e]^T + b[e]
 * [P2 "主張と根拠": the ragged groups of all experts in one grouped-GEMM
 * call; P1 "MoE ブロックにおけるトレーニングのボトルネック克服": FC2 of the
 * expert MLP, and the GroupGemm + Quantize family for the MX output option
 * below].  Row r belongs to the expert e whose segment holds it.
 *   a [R, K] dtype;  w [E, N, K] dtype;  b [E, N] float32 nullable;
 *   y [R, N] dtype.  (FC2: K = f, N = d.)
 * Argument errors (null or misaligned pointers, N or K not a multiple of 8)
 * return MOE_ERR_INVALID_ARG before anything is enqueued. */
typedef struct {
  size_t struct_size; /* = sizeof(moe_gemm_fwd_args_t) */
  int dtype;
  const void* a;
  const void* w;
  const float* b;
  const int32_t* offsets;
  int E, R, N, K;
  void* y;
  int max_cus;
  /* dtype == MOE_E4M3 or MOE_E2M1: a_mx [R, K] and w_mx [E*N, K] row copies replace a / w;
   * y is bf16; no bias. */
  const moe_mx_t* a_mx;
  const moe_mx_t* w_mx;
  /* MX operands only (nullable): y written as an MX row copy [R, N] in the
   * operands' element format (blocks along N, quantized from the float32
   * products; N a multiple of 32) instead of bf16 -- the quantized GEMM
   * output of a low-precision dispatch; y may then be NULL. */
  moe_mx_t* y_mx;
} moe_gemm_fwd_args_t;
moe_status_t moe_grouped_gemm_fwd(const moe_gemm_fwd_args_t* args, void* stream);

/* a8.  FC2 dgrad with the dGLU epilogue [P1 "融合された GEMM エピローグ…":
 * the backward epilogue reads the GEMM output and computes dSwiGLU]:
 *   dA[r] = dy[r] @ w2[e]                        (float32 accumulate)
 *   dH    = (dA * lin * act'(gate) * [gate <= L],  dA * act(gate) * [|lin| <= L])
 * written in the packed column layout of h (for SRELU: dH = dA * 2 relu(h) * [h <= L]).
 *   dy [R, d] dtype;  w2 [E, d, f] dtype;  h [R, n1] dtype (saved by FC1);
 *   dh [R, n1] dtype (out). */
typedef struct {
  size_t struct_size; /* = sizeof(moe_glu_bwd_args_t) */
  int dtype;
  const void* dy;
  const void* w2;
  const void* h;
  const int32_t* offsets;
  int E, R, d, f;
  int act;
  float clamp;
  float alpha;
  int gelu_tanh;
  void* dh;
  int max_cus;
  /* dtype == MOE_E4M3 or MOE_E2M1: dy_mx [R, d] (row copy along d) and w2t_mx [E*f, d]
   * (W2 transposed, blocked along d) replace dy / w2; h is bf16; dH is written
   * as dh_row (row copy [R, n1] in the packed layout, nullable) and dh_col
   * (column copy [n1, moe_mx_col_len], nullable, needs pad_offsets), quantized
   * from the float32 epilogue values.  Gated activations only. */
  const moe_mx_t* dy_mx;
  const moe_mx_t* w2t_mx;
  moe_mx_t* dh_row;
  moe_mx_t* dh_col;
  const int32_t* pad_offsets;
  /* bf16 / float32 (nullable): W2 transposed, w2t [E, f, d] with
   * w2t[e][j][i] == w2[e][i][j] (moe_transpose_weights).  When set it is read
   * instead of w2 (which may then be NULL), K-contiguous like dy. */
  const void* w2t;
  /* Feature scaling (every dtype; see moe_glu_fwd_args_t.row_scale):
   *   row_scale   [R] float32 (in, nullable): the activation's gradient is
   *               taken at row_scale[r] * dA[r];
   *   d_row_scale [R] float32 (out, nullable): the factor's gradient
   *               ds[r] = sum_c dA[r,c] * act(H[r])[c]  (act of the stored H,
   *               clamp included; unscaled dA), zero for rows at or past
   *               offsets[E];
   *   ws, ws_bytes: device workspace of at least
   *               moe_glu_bwd_workspace_size(R, f) bytes, needed with
   *               d_row_scale (else MOE_ERR_WORKSPACE): the epilogue writes
   *               one partial sum per 32 columns of dA and row there, and a
   *               second kernel adds them in column order (deterministic, no
   *               atomics). */
  const float* row_scale;
  float* d_row_scale;
  void* ws;
  size_t ws_bytes;
} moe_glu_bwd_args_t;
moe_status_t moe_grouped_gemm_glu_bwd(const moe_glu_bwd_args_t* args, void* stream);
size_t moe_glu_bwd_workspace_size(int R, int f);

/* a9 / a10 / a11.  Backward of the grouped linear map y = a @ w[e]^T (+ b[e])
 * [P1 "融合された GEMM エピローグによる GLU 活性化関数の最適化": the backward
 * pass of the expert MLP's grouped GEMMs (FC2's weight gradient, FC1's input
 * and weight gradients); P2 "主張と根拠": one call over all ragged expert
 * groups, the weight gradient reducing over each expert's rows]:
 *   DGRAD: da[r] = g[r] @ w[e]                 g [R, N], w [E, N, K] dtype,
 *          da [R, K] dtype (out).
 *   WGRAD: dw[e] = g[seg e]^T @ a[seg e]       g [R, N], a [R, K] dtype,
 *          dw [E, N, K] float32 (out; exact zeros for empty experts; added to
 *          the existing values when `accumulate`), db [E, N] float32
 *          (out, nullable): column sums of g over each segment (added to
 *          the existing values when `accumulate`, like dw). */
typedef struct {
  size_t struct_size; /* = sizeof(moe_gemm_bwd_args_t) */
  int dtype;
  int mode;            /* moe_bwd_mode_t */
  const void* g;
  const void* a;       /* WGRAD */
  const void* w;       /* DGRAD */
  const int32_t* offsets;
  int E, R, N, K;
  void* out;           /* da (DGRAD) or dw (WGRAD) */
  float* db;           /* WGRAD, nullable */
  int accumulate;
  int max_cus;
  /* dtype == MOE_E4M3 or MOE_E2M1:
   *   DGRAD: g_mx [R, N] row copy, w_mx [E*K, N] (w transposed, blocked along
   *          N); da is bf16.
   *   WGRAD: g_mx [N, L] and a_mx [K, L] column copies (L = moe_mx_col_len),
   *          segments from pad_offsets; dw float32; db must be NULL. */
  const moe_mx_t* g_mx;
  const moe_mx_t* a_mx;
  const moe_mx_t* w_mx;
  const int32_t* pad_offsets;
  /* WGRAD, gather-fused permute (bf16 / float32; nullable): with a_src_row
   * from moe_permute, a is the unpermuted [a_src_rows, K] and row r of the
   * segments reads a[a_src_row[r]] (FC1's weight gradient straight from x).
   * Same limits as moe_glu_fwd_args_t.src_row. */
  const int32_t* a_src_row;
  int a_src_rows;
  /* DGRAD with MX operands (nullable): da written as an MX row copy [R, K]
   * in the operands' element format (blocks along K, from the float32
   * products; K a multiple of 32) instead of bf16, e.g. dXp for a quantized
   * dispatch backward (moe_unpermute_combine_mx sums it); out may then be
   * NULL. */
  moe_mx_t* out_mx;
  /* DGRAD, bf16 / float32 (nullable): w transposed, wt [E, K, N] with
   * wt[e][j][i] == w[e][i][j] (moe_transpose_weights).  When set it is read
   * instead of w (which may then be NULL), K-contiguous like g. */
  const void* wt;
} moe_gemm_bwd_args_t;
moe_status_t moe_grouped_gemm_bwd(const moe_gemm_bwd_args_t* args, void* stream);

/* ---------------------------------------------------------------- MXFP8 (a14)
 * [P1] section "MXFP8 および NVFP4 量子化の融合による露出メモリオーバーヘッドの削減":
 * GEMM outputs are quantized to MXFP8 inside the kernels that produce them,
 * together with a transposed copy for the backward pass, so quantization
 * costs no separate pass over memory.  Format: OCP Microscaling Formats (MX)
 * v1.0 -- E4M3 elements (largest magnitude 448, no infinities) and one E8M0
 * scale 2^(code - 127) per 32 consecutive elements of a row; a block with
 * largest magnitude amax has shared exponent e = floor(log2 amax) - 8,
 * clamped to [-127, 127] (amax = 0: e = -127), and elements
 * round_to_nearest_even(v / 2^e) saturated to +-448.
 *
 * A quantized matrix is a moe_mx_t: `data` [rows, ld] E4M3 codes, `scale`
 * [rows, ld / 32] E8M0 codes (scale[r * ld/32 + b] covers data[r*ld + 32b ..
 * 32b + 31]), ld a multiple of 32.  Every GEMM operand is blocked along that
 * GEMM's reduction axis, so each operand is a K-contiguous MX matrix:
 *  - row copy of X [R, n]: rows = R, ld = n (blocks along the features);
 *  - column copy of X [R, n] split into expert segments: rows = n, ld =
 *    moe_mx_col_len(R, E); expert e's tokens occupy [pad_offsets[e],
 *    pad_offsets[e+1]) of every row (the segment start anchors the 32-blocks,
 *    the tail of the last block is zero); entries past pad_offsets[E] are not
 *    written;
 *  - weight copies: W [E, N, K] blocked along K is a row copy with rows E*N,
 *    ld = K; blocked along N it is the transposed copy [E*K rows, ld = N].
 * MX GEMM operands need the reduction length (K, ld) a multiple of 128.
 * The layer's MXFP8 variant has no biases.  (moe_mx_t is declared beside the
 * element types above.)
 *
 * MXFP4 (dtype MOE_E2M1, the 4-bit variant; the pages' 4-bit format is NVFP4,
 * whose E2M1 elements the CDNA4 matrix cores take with E8M0 scales per 32):
 * the same layouts with E2M1 elements -- sign, 2 exponent bits, 1 mantissa
 * bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 -- packed two per byte (element
 * 2i in the low nibble of byte i, so a row holds ld / 2 bytes), block
 * exponent e = floor(log2 amax) - 2, elements rounded to nearest even and
 * saturated to +-6 (a NaN becomes +-6).  The GEMM entry points take MXFP4
 * operands with dtype MOE_E2M1 and write their MX outputs (A, dH copies) in
 * MXFP4 too; the moe_mxfp4_quantize* functions mirror the MXFP8 ones. */

/* Length of the token axis of an expert-segmented column copy:
 * R + 31 E rounded up to a multiple of 128 (an upper bound of pad_offsets[E]). */
int64_t moe_mx_col_len(int R, int E);

/* Leading dimension to allocate a column copy with (elements, >= the
 * length above): the smallest one whose row stride in bytes is an odd
 * multiple of 128 (dtype MOE_E4M3 or MOE_E2M1; 0 for another dtype).  The
 * weight-gradient GEMMs read 128 bytes of many rows at once; with a row
 * stride of an even multiple of 128 bytes (the length above at most
 * workload shapes) those reads fall on few HBM channels and run slower. */
int64_t moe_mx_col_ld(int R, int E, int dtype);

/* Row copy: out = MX(x) along the last axis.  x [rows, n] dtype (F32 or BF16),
 * n a multiple of 32; out->data [rows, out->ld >= n], blocks along n. */
moe_status_t moe_mx_quantize(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                             void* stream);

/* Transposed copy of a batch of matrices: x [batches, rows, n] dtype, rows a
 * multiple of 32; out row b*n + c holds column c of matrix b, blocked along
 * rows: out->data [batches * n, out->ld >= rows]. */
moe_status_t moe_mx_quantize_transpose(const void* x, int dtype, int batches, int rows, int n,
                                       moe_mx_t* out, void* stream);

/* Row and/or column copies of an expert-ordered tensor, read straight from
 * its source rows (a2 and a6 fused with the quantization):
 *   v[r][c] = x[src_row ? src_row[r] : r][c] * (topk_w ? topk_w[t*k + j] : 1)
 * where t = src_row[r] and row_map[t*k + j] = r (float32 product).  With
 * src_row = x's permutation this is Xp; with x = d_out and the gates it is
 * dY = w * dOut.  x [*, n] dtype; src_row, offsets, pad_offsets from
 * moe_permute; row_map and topk_w required together, and only with src_row.
 *   row_out (nullable): [R, ld >= n] blocks along n;
 *   col_out (nullable): [n, moe_mx_col_len(R, E)] blocks along tokens. */
moe_status_t moe_mx_quantize_experts(const void* x, int dtype, const int32_t* src_row,
                                     const int32_t* row_map, const float* topk_w, int k,
                                     const int32_t* offsets, const int32_t* pad_offsets, int E,
                                     int R, int n, moe_mx_t* row_out, moe_mx_t* col_out,
                                     void* stream);

/* MXFP4 counterparts of the three quantizers above (same arguments; out,
 * row_out, col_out receive E2M1 codes, ld / 2 bytes per row). */
moe_status_t moe_mxfp4_quantize(const void* x, int dtype, int64_t rows, int n, moe_mx_t* out,
                                void* stream);
moe_status_t moe_mxfp4_quantize_transpose(const void* x, int dtype, int batches, int rows, int n,
                                          moe_mx_t* out, void* stream);
moe_status_t moe_mxfp4_quantize_experts(const void* x, int dtype, const int32_t* src_row,
                                        const int32_t* row_map, const float* topk_w, int k,
                                        const int32_t* offsets, const int32_t* pad_offsets, int E,
                                        int R, int n, moe_mx_t* row_out, moe_mx_t* col_out,
                                        void* stream);

/* ---------------------------------------------------------------- combine
 * a5 / a12.  The weighted combine that closes the MoE layer ([P3] "FlashMoE:
 * Fast Distributed MoE in a Single Kernel", Abstract, names the dispatch,
 * compute and combine phases of a MoE operator; P2 "主張と根拠" the combine
 * that collects the experts' results).  The pages do not define it; the
 * reading taken here is the usual gate-weighted sum, deterministic:
 *   out[t] = sum_{j=0..k-1} topk_w[t,j] * y[row_map[t,j]], summed in float32
 * in slot order and rounded once, no atomics (topk_w NULL: unit weights, the
 * unpermute-sum of the backward).  y [T*k, d] dtype; out [T, d] dtype;
 * row_map [T, k] from moe_permute.  Argument errors (null or misaligned
 * pointers, d * element size not a multiple of 16) return a status code. */
moe_status_t moe_unpermute_combine(const void* y, int dtype, const int32_t* row_map,
                                   const float* topk_w, int T, int k, int d, void* out,
                                   void* stream);

/* a12 from MX rows: out[t] = sum_{j<k} (topk_w ? topk_w[t,j] : 1) * decode(y)[row_map[t,j]],
 * decode(y) = codes x block scale, summed in float32 in slot order, rounded
 * once to out_dtype (F32 or BF16).  y [T*k, d] MX row copy of element format
 * y_dtype (MOE_E4M3 or MOE_E2M1), d a multiple of 32; out [T, d]. */
moe_status_t moe_unpermute_combine_mx(const moe_mx_t* y, int y_dtype, const int32_t* row_map,
                                      const float* topk_w, int T, int k, int d, void* out,
                                      int out_dtype, void* stream);

/* a6.  Backward of the combine (the exact gradient of the reading stated at
 * moe_unpermute_combine; pages as there):
 *   d_y[row_map[t,j]]  = topk_w[t,j] * d_out[t]        (dtype, rounded once)
 *   d_topk_w[t,j]      = <d_out[t], y[row_map[t,j]]>   (float32, summed in a
 *                        fixed order)
 * d_out [T, d], y [T*k, d], d_y [T*k, d] dtype.  d_y or d_topk_w may be NULL
 * (an MXFP8 layer writes dY only as MXFP8 copies, with moe_mx_quantize_experts).
 * topk_w NULL: unit weights (the combine of a layer whose gates scale FC1's
 * activation); y is read only for d_topk_w and may be NULL without it. */
moe_status_t moe_unpermute_combine_bwd(const void* d_out, const void* y, int dtype,
                                       const int32_t* row_map, const float* topk_w, int T,
                                       int k, int d, void* d_y, float* d_topk_w, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
