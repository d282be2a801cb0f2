// Ragged grouped GEMMs of the expert FFN, with fused epilogues.
//
// [P2] "JAXとNVIDIA Transformer EngineによるDropless MoE学習の高速化", section
// "主張と根拠": all ragged expert groups are multiplied in one kernel call.
// [P1] "高度な融合カーネルによる MoE 学習スループットの向上":
//  - "ホストとデバイスの同期および CPU 起動オーバーヘッドの排除": the kernel reads
//    the rows per group from GPU memory, so the launch needs no host-side shape
//    and the layer can be captured in a graph;
//  - "融合された GEMM エピローグによる GLU 活性化関数の最適化" (+ Figure 2): with
//    the FC1 weights repacked into interleaved gate / linear column chunks, the
//    tile that computes a gate column also computes the matching linear
//    column, so the GLU is applied in registers in the epilogue; the backward
//    epilogue reads the saved pre-activation and applies dGLU;
//  - "カーネルレベルでの向上から事前学習全体の速度向上へ": dynamic scheduling
//    and a limit on the compute units a kernel occupies.
//
// Design (gfx950 / CDNA4):
//  * Persistent launch: grid = (compute units) x (resident workgroups per
//    CU).  Each workgroup reads offsets[E+1] once, builds the tile table in
//    LDS and takes one tile per round, r * grid + vb.  The virtual id vb
//    groups consecutive tiles on one XCD (blocks are dealt round-robin over
//    the 8 XCDs), and tiles are ordered in bands of GM M-tiles (default 4)
//    so the workgroups of an XCD share A rows and B columns in its L2.
//  * Two grouping modes: RAGGED_M (FC1, FC2, dgrads: M = rows of an expert,
//    B = that expert's weight) and RAGGED_K (weight gradients: K = rows of an
//    expert; experts visited largest first so the long tiles start early,
//    and odd rounds run backwards to even out the per-block sums).
//  * Tiles of BM x BN x (128 bytes of K) in a ring of LDS stages, filled by
//    LDS-DMA loads (buffer_load ... lds, no staging registers).  A
//    K-contiguous operand keeps 128 bytes of K per LDS row, 16-byte chunk c
//    of row r at slot c ^ ((r >> 1) & 7), so fragment reads touch every bank
//    once.  An MN-contiguous operand (the transposed operand of a dgrad or
//    weight gradient) keeps one k per LDS row and is read with
//    ds_read_b64_tr_b16, which hands each lane the k-run its MFMA fragment
//    needs.
//  * MFMA v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32),
//    fp32 accumulation.  The MFMA is issued with B as the first operand, so a
//    lane's 16 accumulators hold 4 runs of 4 consecutive output columns of one
//    row: the epilogue writes 8- or 16-byte vectors, and the gate and linear
//    halves of a GLU pair sit in the same lane at the same positions.
#include "common.hpp"
#include "mx.hpp"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#include <type_traits>

namespace moe {

// Epilogues.  The activation is part of the id, so each kernel carries the
// code of one activation only.
enum {
  EPI_STORE = 0,       // C = acc (+ bias)                     (plain grouped GEMM / dgrad / wgrad)
  EPI_SWIGLU_FWD = 1,  // H = acc + b1;  A = silu_a(gate) * lin (FC1)
  EPI_GEGLU_FWD = 2,   // H = acc + b1;  A = gelu(gate) * lin   (FC1)
  EPI_SRELU_FWD = 3,   // H = acc + b1;  A = relu(h)^2          (FC1, not gated)
  EPI_SWIGLU_BWD = 4,  // dH from dA = acc and the saved H       (FC2 dgrad)
  EPI_GEGLU_BWD = 5,
  EPI_SRELU_BWD = 6
};
constexpr bool epi_glu_fwd(int e) { return e == EPI_SWIGLU_FWD || e == EPI_GEGLU_FWD; }
constexpr bool epi_glu_bwd(int e) { return e == EPI_SWIGLU_BWD || e == EPI_GEGLU_BWD; }
enum { RAGGED_M = 0, RAGGED_K = 1 };

// MXFP8 operands: E4M3 codes (16 per 16-byte chunk) with one E8M0 scale per
// 32 along K, multiplied by v_mfma_scale_f32_32x32x64_f8f6f4.  Both operands
// are K-contiguous; outputs of these GEMMs are bf16 (or float32 for weight
// gradients, or MXFP8 copies written by the epilogue).
// MX operands: EPB k elements per storage byte, FMT the scaled MFMA's
// operand format code (0 = E4M3, 4 = E2M1).  The loaders count K in bytes.
struct MX8 {
  typedef uint8_t storage;
  static constexpr int VEC = 16;
  static constexpr int EPB = 1, FMT = 0;
  typedef FmtE4M3 Fmt;
};
struct MX4 {
  typedef uint8_t storage;
  static constexpr int VEC = 16;
  static constexpr int EPB = 2, FMT = 4;
  typedef FmtE2M1 Fmt;
};
template <class EL>
constexpr bool is_mx() {
  return std::is_same<EL, MX8>::value || std::is_same<EL, MX4>::value;
}
template <class EL>
constexpr int epb() {
  if constexpr (is_mx<EL>()) return EL::EPB;
  else return 1;
}
// storage type of the GEMM's own outputs (C, saved H)
template <class EL>
struct OutT {
  typedef typename EL::storage type;
};
template <>
struct OutT<MX4> {
  typedef uint16_t type;
};
template <>
struct OutT<MX8> {
  typedef uint16_t type;
};

struct GemmArgs {
  const void* a;
  const void* b;
  const int32_t* offsets;
  int E, R;
  int M, N, K;  // RAGGED_M: N, K used (M ragged); RAGGED_K: M, N used (K ragged)
  long long lda, ldb, ldc, ld_aux;
  long long b_expert_stride;  // RAGGED_M: elements between experts' B
  long long c_expert_stride;  // RAGGED_K: elements between experts' C
  void* c;
  const float* bias;  // RAGGED_M: [E][ld_bias]
  long long ld_bias;
  void* aux;  // GLU/SRELU forward: saved pre-activation (nullable); backward: input H
  float clamp, alpha;
  int act, gelu_tanh;
  int accumulate;
  int gm;    // M-tiles per band of the tile order (RAGGED_M)
  int gm_k;  // the same for the weight gradients (RAGGED_K)
  int snake;  // RAGGED_K: odd rounds of the tile order run backwards
  int glu_direct;  // tuning builds only: FC1 + GLU stores without the LDS staging (1), or A's (2)
  // Gather-fused permute (nullable): RAGGED_M reads row r of A as row
  // gather[r] of a; RAGGED_K reads k-row r of B as row gather[r] of b; the
  // gathered source has gather_rows rows.
  const int32_t* gather;
  long long gather_rows;
  // MXFP8 operands (MX8): E8M0 scales of A and B, row strides in bytes
  const uint8_t* sa;
  const uint8_t* sb;
  long long slda, sldb;
  long long sb_expert_stride;  // RAGGED_M: bytes between experts' B scales
  // MXFP8 copies of the epilogue's output (A of FC1, dH of the dGLU):
  // row copy [R, ld_mxr] and expert-segmented column copy [n, ld_mxc]
  uint8_t* mxr;
  uint8_t* mxr_s;
  long long ld_mxr;
  uint8_t* mxc;
  uint8_t* mxc_s;
  long long ld_mxc;
  const int32_t* pad_offsets;
  // Feature scaling of the GLU / sReLU output (nullable): forward A[r] =
  // row_scale[r] * act; backward the activation's gradient is taken at
  // row_scale[r] * dA, and (ds_part non-null) each 32 x 32 block of dA adds
  // its rows' sum of dA * act into ds_part[(col / 32) * ld_ds + r].
  const float* row_scale;
  float* ds_part;
  long long ld_ds;
};

// ------------------------------------------------------------------ activations

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal
// (relative error about 1e-6 for |x| <= 20; exact limits 0 and 1 outside).
__device__ __forceinline__ float sigm(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// Activation value and derivative.  GATED_SWIGLU: silu_a(g) = g sigmoid(a g);
// GATED_GEGLU: g Phi(g) (erf form) or its tanh approximation; SRELU: relu(g)^2.
enum { ACT_SWIGLU = 0, ACT_GEGLU = 1, ACT_SRELU = 2 };

template <int ACT>
__device__ __forceinline__ float act_value(float g, float alpha, int gtanh) {
  if constexpr (ACT == ACT_SWIGLU) {
    return g * sigm(alpha * g);
  } else if constexpr (ACT == ACT_GEGLU) {
    if (gtanh) {
      const float c = 0.7978845608028654f;
      return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
    }
    return 0.5f * g * (1.0f + erff(g * 0.7071067811865476f));
  } else {
    float r = fmaxf(g, 0.0f);
    return r * r;
  }
}

template <int ACT>
__device__ __forceinline__ void act_value_grad(float g, float alpha, int gtanh, float& a,
                                               float& da) {
  if constexpr (ACT == ACT_SWIGLU) {
    const float sg = sigm(alpha * g);
    a = g * sg;
    da = sg + alpha * g * sg * (1.0f - sg);
  } else if constexpr (ACT == ACT_GEGLU) {
    if (gtanh) {
      const float c = 0.7978845608028654f;
      const float th = tanhf(c * (g + 0.044715f * g * g * g));
      a = 0.5f * g * (1.0f + th);
      da = 0.5f * (1.0f + th) + 0.5f * g * (1.0f - th * th) * c * (1.0f + 0.134145f * g * g);
    } else {
      const float cdf = 0.5f * (1.0f + erff(g * 0.7071067811865476f));
      a = g * cdf;
      da = cdf + g * expf(-0.5f * g * g) * 0.3989422804014327f;
    }
  } else {
    const float r = fmaxf(g, 0.0f);
    a = r * r;
    da = 2.0f * r;
  }
}

constexpr int epi_act(int e) {
  return (e == EPI_GEGLU_FWD || e == EPI_GEGLU_BWD) ? ACT_GEGLU
         : (e == EPI_SRELU_FWD || e == EPI_SRELU_BWD) ? ACT_SRELU : ACT_SWIGLU;
}

// ------------------------------------------------------------------ tile loaders

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Byte offset that a buffer access treats as out of range (it returns zeros).
static constexpr uint32_t OOB = 0x80000000u;

// Operand tiles go global -> LDS directly (buffer_load ... lds, 16 bytes per
// lane): no staging registers, and elements outside the operand (rows past a
// segment end, columns past N, k past K) read as zeros through the buffer
// range check instead of branches.  A wave instruction fills 1 KB of LDS;
// each lane chooses which 16-byte global chunk lands in its 16 LDS bytes,
// which is how the swizzled LDS layouts below are produced.
//
// Interface of both loaders: setup(X, ld, mn0, mnlim, kend, tid) once per
// tile, issue(stage, k0) once per k-step of 128 bytes of K.

// K-contiguous operand X[mn][k]: LDS row = one mn index holding BKB bytes of
// K as CPR = BKB / 16 chunks of 16 bytes; chunk c of row r sits at slot
// c ^ ((r >> RSH) & (CPR - 1)), RSH = log2(256 / BKB).  The 64 banks span 256
// bytes, i.e. 256 / BKB rows.  A fragment read serves 16 lanes per LDS cycle,
// one chunk of 16 consecutive rows: rows in the same 256-byte window sit at
// different offsets in it, and rows of different windows get different XOR
// keys, so the 16 lanes touch 16 distinct 16-byte bank groups.
template <int BKB>
struct KGeom {
  static constexpr int CPR = BKB / 16;             // chunks per row
  static constexpr int RPI = 1024 / BKB;           // rows per wave DMA instruction
  static constexpr int RSH = BKB == 128 ? 1 : 2;   // log2(rows per 256-byte window)
  static_assert(BKB == 64 || BKB == 128, "64- or 128-byte k steps");
  __device__ __forceinline__ static int slot(int row, int chunk) {
    return chunk ^ ((row >> RSH) & (CPR - 1));
  }
};

template <class EL, int ROWS, int THREADS, int BKB, bool GATHER = false>
struct DmaK {
  typedef typename EL::storage S;
  typedef KGeom<BKB> Gm;
  static constexpr int NW = THREADS / 64;
  static constexpr int PER = ROWS / Gm::RPI / NW;   // wave instructions per step
  static_assert(ROWS % (Gm::RPI * NW) == 0, "rows must split evenly over the waves");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[PER];
  int kc[PER];
  int K, Klo;

  // GATHER: row r of the operand is row gidx[r] of X, which has grows rows
  // (gather-fused permute); X then spans at most 2 GiB.
  __device__ __forceinline__ void setup(const S* X, long long ld, int r0, int rlim, int Kdim,
                                        int tid, int Kmin = 0, const int32_t* gidx = nullptr,
                                        long long grows = 0) {
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    K = Kdim;
    Klo = Kmin;
    if constexpr (GATHER) {
      const long long bytes = grows * ld * (long long)sizeof(S);
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<S*>(X), (short)0,
                                             (int)(bytes > 0x7ffffff0LL ? 0x7ffffff0LL : bytes),
                                             0x00020000);
    } else {
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<S*>(X) + (size_t)r0 * ld, (short)0,
                                             0x7ffffff0, 0x00020000);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      // lane l fills slot l % CPR of row l / CPR of this instruction's rows
      const int row = Gm::RPI * (w * PER + i) + lane / Gm::CPR;
      const int c = Gm::slot(row, lane % Gm::CPR);    // the chunk that belongs there
      kc[i] = c * EL::VEC;
      if constexpr (GATHER) {
        const int src = (r0 + row < rlim) ? gidx[r0 + row] : -1;
        voff[i] = (src >= 0 && src < grows) ? (uint32_t)(((size_t)src * ld + kc[i]) * sizeof(S))
                                            : OOB;
      } else {
        voff[i] = (r0 + row < rlim) ? (uint32_t)(((size_t)row * ld + kc[i]) * sizeof(S)) : OOB;
      }
    }
  }
  __device__ __forceinline__ void issue(u32x4* stage, int k0) const {
    // the LDS destination (M0) must be wave-uniform: derive the wave id so the
    // compiler can see that
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kk = k0 + kc[i];
      const uint32_t kbad = (kk < K && kk >= Klo) ? 0u : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(stage + (w * PER + i) * 64), 16,
                                               (int)(voff[i] | kbad), k0 * (int)sizeof(S), 0, 0);
    }
  }
};

// MN-contiguous operand X[k][mn]: LDS row = one k index holding the tile's
// ROWS values of mn.  For bf16, 16-byte chunk c of k-row k sits at slot
// c ^ ((k & 3) << 2): the transposed fragment reads below touch 4 consecutive
// k-rows x 64 bytes per half wave, which this spreads over distinct banks.
template <class EL, int ROWS, int THREADS, int BKB, bool GATHER = false>
struct DmaMN {
  typedef typename EL::storage S;
  static constexpr int V = EL::VEC;
  static constexpr int ROWB = ROWS * (int)sizeof(S);   // bytes per k-row
  static constexpr int BK = BKB / (int)sizeof(S);       // k-rows per step
  static constexpr int INSTR = BK * ROWB / 1024;
  static constexpr int NW = THREADS / 64;
  static constexpr int PER = INSTR / NW;
  static constexpr int RPI = 1024 / ROWB;                // k-rows per wave instruction
  static constexpr bool SWZ = sizeof(S) == 2;
  static_assert(ROWB <= 1024 && INSTR % NW == 0, "tile does not split into wave loads");
  static_assert(!SWZ || ROWB % 256 == 0, "the bf16 swizzle needs 16 chunks per k-row");
  static constexpr int KPW = PER * RPI;                 // consecutive k-rows per wave
  typedef __attribute__((address_space(4))) const int32_t* CIdx;
  const S* X;
  long long ld;
  int c0, clim, kend, krl, slot;
  // Gather-fused permute (GATHER): k-row k is row gidx[k] of X.  The
  // source rows of the wave's KPW k-rows of the next step to be issued are
  // read ahead with scalar loads (the same for every lane), so a step's DMA
  // never waits on its index fetch; steps are issued in increasing order.
  CIdx gidx;
  __amdgpu_buffer_rsrc_t grs;
  int gn;  // rows of X
  int gi[KPW];

  __device__ __forceinline__ void fetch_rows(int k0) {
    const int base = k0 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * KPW;
#pragma unroll
    for (int q = 0; q < KPW; ++q) gi[q] = gidx[max(min(base + q, kend - 1), 0)];
  }

  // Kmin: the first k of the first step (steps follow at BK intervals).
  // gidx / grows: gathered source (rows of X), nullable.
  __device__ __forceinline__ void setup(const S* X_, long long ld_, int c0_, int clim_, int kend_,
                                        int tid, int Kmin = 0, const int32_t* gidx_ = nullptr,
                                        long long grows = 0) {
    X = X_;
    ld = ld_;
    c0 = c0_;
    clim = clim_;
    kend = kend_;
    const int lane = tid & 63;
    krl = (16 * lane) / ROWB;
    slot = ((16 * lane) % ROWB) / 16;
    if constexpr (GATHER) {
      gidx = (CIdx)gidx_;
      long long bytes = (grows * ld - c0) * (long long)sizeof(S);
      bytes = bytes < 0 ? 0 : (bytes > 0x7ffffff0LL ? 0x7ffffff0LL : bytes);
      gn = (int)grows;
      grs = __builtin_amdgcn_make_buffer_rsrc(const_cast<S*>(X) + c0, (short)0, (int)bytes,
                                              0x00020000);
      if (Kmin < kend) fetch_rows(Kmin);
    }
  }
  __device__ __forceinline__ void issue(u32x4* stage, int k0) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int kr = (w * PER + i) * RPI + krl;
        const int chunk = SWZ ? (slot ^ ((kr & 3) << 2)) : slot;
        int src = gi[i * RPI];
#pragma unroll
        for (int r = 1; r < RPI; ++r) src = krl == r ? gi[i * RPI + r] : src;
        const bool ok = (k0 + kr < kend) && (c0 + chunk * V < clim) && src >= 0 && src < gn;
        const uint32_t vo = ok ? (uint32_t)(((size_t)src * ld + chunk * V) * sizeof(S)) : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, LDS_PTR(stage + (w * PER + i) * 64), 16,
                                                 (int)vo, 0, 0, 0);
      }
      if (k0 + BK < kend) fetch_rows(k0 + BK);
      return;
    }
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S*>(X) + (size_t)k0 * ld + c0, (short)0, 0x7ffffff0, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kr = (w * PER + i) * RPI + krl;
      const int chunk = SWZ ? (slot ^ ((kr & 3) << 2)) : slot;
      const bool ok = (k0 + kr < kend) && (c0 + chunk * V < clim);
      const uint32_t vo = ok ? (uint32_t)(((size_t)kr * ld + chunk * V) * sizeof(S)) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(stage + (w * PER + i) * 64), 16,
                                               (int)vo, 0, 0, 0);
    }
  }
};

// MFMA fragment of 32 mn-rows starting at r0, k sub-step s of a step (16 k for
// bf16, 8 k for fp32; BKB / 32 sub-steps): lane l holds mn = r0 + (l & 31) and
// the 16-byte k-chunk 2 s + (l >> 5).
template <bool KMAJ, class EL, int ROWS, int BKB>
struct Frag;

template <class EL, int ROWS, int BKB>
struct Frag<true, EL, ROWS, BKB> {
  static constexpr int READS = 1;  // LDS read instructions per fragment
  __device__ __forceinline__ static u32x4 load(const u32x4* st, int r0, int s, int lane) {
    typedef KGeom<BKB> Gm;
    const int row = r0 + (lane & 31), ch = 2 * s + (lane >> 5);
    return st[row * Gm::CPR + Gm::slot(row, ch)];
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

// bf16 from a [k][mn] tile with ds_read_b64_tr_b16.  Within each group of 16
// lanes, lane i receives element (i mod 4) of the 8-byte segments addressed by
// lanes 4 q + i / 4, q = 0..3.  Lane j = 16 g + 4 q + r therefore addresses
// k-row kb + q, mn columns mb + 4 r .. + 3, so that every lane i of the group
// ends up with k = kb .. kb + 3 of mn = mb + i: half of its MFMA fragment.
template <int ROWS, int BKB>
struct Frag<false, BF16, ROWS, BKB> {
  static constexpr int READS = 2;
  __device__ __forceinline__ static u32x4 load(const u32x4* st, int r0, int s, int lane) {
    constexpr int ROWB = ROWS * 2;
    const int g = lane >> 4, q = (lane >> 2) & 3, r = lane & 3;
    const int mn = r0 + 16 * (g & 1) + 4 * r;
    const char* base = reinterpret_cast<const char*>(st);
    u32x4 out;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = 16 * s + 8 * (g >> 1) + 4 * half + q;
      const int chunk = (mn >> 3) ^ (q << 2);  // k & 3 == q
      const char* p = base + k * ROWB + chunk * 16 + (mn & 7) * 2;
      i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p));
      u32x2 w = __builtin_bit_cast(u32x2, v);
      out[2 * half] = w[0];
      out[2 * half + 1] = w[1];
    }
    return out;
  }
};

// fp32 from a [k][mn] tile: the fp32 MFMA takes one value per lane, element q
// of the lane's k-chunk, i.e. k = 4 (2 s + (l >> 5)) + q.
template <int ROWS, int BKB>
struct Frag<false, F32, ROWS, BKB> {
  static constexpr int READS = 4;
  __device__ __forceinline__ static u32x4 load(const u32x4* st, int r0, int s, int lane) {
    const float* base = reinterpret_cast<const float*>(st);
    const int col = r0 + (lane & 31), kb = 4 * (2 * s + (lane >> 5));
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(base[(kb + q) * ROWS + col]);
    return out;
  }
};

// E8M0 scales of one k-step (128 k = 4 blocks = one 4-byte word per row) for
// the BM rows of A and then the BN rows of B: (BM + BN) / 64 dword DMA
// instructions, one per wave; word r of the stage's scale area belongs to row r.
template <int BM, int BN, int THREADS>
struct DmaScale {
  static_assert((BM + BN) / 64 == THREADS / 64, "one scale load per wave");
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff;

  __device__ __forceinline__ void setup(const uint8_t* sa, long long slda, int m0, int mlim,
                                        const uint8_t* sb, long long sldb, int n0, int N,
                                        int tid) {
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t* base;
    if (w * 64 < BM) {
      const int row = w * 64 + lane;
      base = sa + (size_t)m0 * slda;
      voff = (m0 + row < mlim) ? (uint32_t)((size_t)row * slda) : OOB;
    } else {
      const int row = w * 64 - BM + lane;
      base = sb + (size_t)n0 * sldb;
      voff = (n0 + row < N) ? (uint32_t)((size_t)row * sldb) : OOB;
    }
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7ffffff0,
                                           0x00020000);
  }
  __device__ __forceinline__ void issue(uint32_t* scales, int k0) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(scales + w * 64), 4, (int)voff, k0 / 32,
                                             0, 0);
  }
};

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// MXFP8 fragment of 32 rows for k sub-step s (64 k) of a 128-byte step.  The
// scaled MFMA takes, per lane of half h = l >> 5, k = 16 h .. 16 h + 15 in
// bytes 0-15 and k = 32 + 16 h .. in bytes 16-31; block 0 (k < 32) is scaled
// by the h = 0 lane's scale, block 1 by the h = 1 lane's (lane layout and
// scale pairing measured on the device).  So the lane reads 16-byte chunks
// 4 s + h and 4 s + 2 + h of its row.
template <int ROWS, int BKB, class EL = MX8>
struct FragMX {
  static constexpr int READS = 2;
  __device__ __forceinline__ static u32x8 load(const u32x4* st, int r0, int s, int lane) {
    typedef KGeom<BKB> Gm;
    const int row = r0 + (lane & 31), h = lane >> 5;
    const u32x4 lo = st[row * Gm::CPR + Gm::slot(row, 4 * s + h)];
    const u32x4 hi = st[row * Gm::CPR + Gm::slot(row, 4 * s + 2 + h)];
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// MXFP4 fragment for k sub-step s (64 k = 32 bytes) of a 64-byte step: with
// E2M1 operands the scaled MFMA reads 16 bytes per lane, lane half h holding
// block h (k = 32 h .. 32 h + 31 of the sub-step) in its first four dwords
// and ignoring the other four (measured on the device), so the lane reads
// chunk 2 s + h of its row.
template <int ROWS, int BKB>
struct FragMX<ROWS, BKB, MX4> {
  static constexpr int READS = 1;
  __device__ __forceinline__ static u32x8 load(const u32x4* st, int r0, int s, int lane) {
    typedef KGeom<BKB> Gm;
    const int row = r0 + (lane & 31), h = lane >> 5;
    const u32x4 c = st[row * Gm::CPR + Gm::slot(row, 2 * s + h)];
    return u32x8{c[0], c[1], c[2], c[3], 0u, 0u, 0u, 0u};
  }
};

// ------------------------------------------------------------------ MFMA step

__device__ __forceinline__ void mma(f32x16& acc, const u32x4& b, const u32x4& a, BF16) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const u32x4& b, const u32x4& a, F32) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[q]), __uint_as_float(a[q]), acc,
                                               0, 0, 0);
}

// Scaled MX MFMA (operand format FMT: 0 E4M3, 4 E2M1); the scale words
// carry the lane's block scale in byte OPSEL (B first, as for bf16).
template <int OPSEL, int FMT = 0>
__device__ __forceinline__ void mma_mx(f32x16& acc, const u32x8& b, const u32x8& a, uint32_t sb,
                                       uint32_t sa) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, b),
                                                        __builtin_bit_cast(i32x8, a), acc, FMT,
                                                        FMT, OPSEL, (int)sb, OPSEL, (int)sa);
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1.  Used where
// accumulators are indexed, so that no index is ever a run-time value (a
// run-time index would move the accumulator array to private memory).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------------------------ epilogues
//
// Each helper handles one 32 x 32 accumulator block of one lane: the lane's
// row, and columns c0 + 8 g + q (g, q = 0..3), acc[4 g + q].  Pointers are
// the lane's row of each tensor; they are distinct tensors (noalias), so the
// compiler may issue every load of a block before its stores.

template <class S>
__device__ __forceinline__ void epi_store(S* __restrict__ C, const float* __restrict__ bias,
                                          const f32x16& acc, int c0, int N) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = acc[4 * g + q] + (bias ? bias[col + q] : 0.0f);
    store4(C + col, v);
  }
}

__device__ __forceinline__ void epi_store_f32(float* __restrict__ C, const f32x16& acc, int c0,
                                              int N, int accumulate) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    float v[4];
    if (accumulate) load4(C + col, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (accumulate ? v[q] : 0.0f) + acc[4 * g + q];
    store4(C + col, v);
  }
}

// FC1 + GLU: gate block (packed columns c0 + ...) and the linear block 32
// columns further; A column of packed gate column c is 32 (c / 64) + c % 64.
template <int ACT, class S>
__device__ __forceinline__ void epi_glu_fwd(S* __restrict__ Hrow, S* __restrict__ Arow,
                                            const float* __restrict__ bias,
                                            const f32x16& accg, const f32x16& accl, int c0,
                                            int N, float L, float alpha, int gtanh, float sc) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    float gv[4], lv[4], o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gv[q] = accg[4 * g + q] + (bias ? bias[col + q] : 0.0f);
      lv[q] = accl[4 * g + q] + (bias ? bias[col + 32 + q] : 0.0f);
    }
    if (Hrow) {
      store4(Hrow + col, gv);
      store4(Hrow + col + 32, lv);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float gt = gv[q], li = lv[q];
      if (L > 0.0f) {
        gt = fminf(gt, L);
        li = fminf(fmaxf(li, -L), L);
      }
      o[q] = act_value<ACT>(gt, alpha, gtanh) * li * sc;
    }
    store4(Arow + (col >> 6) * 32 + (col & 31), o);
  }
}

// Feature-scaling gradient of one 32 x 32 block: the two lanes of a row
// (l and l ^ 32) add their 16-value sums of dA * act, and the first writes
// the block's partial for its row.  Both lanes of a row run this together.
__device__ __forceinline__ void ds_block_store(float* __restrict__ ds_part, long long ld_ds,
                                               int cblock, int row, bool live, float ps) {
  const float tot = ps + __shfl_xor(ps, 32);
  if (live && (threadIdx.x & 32) == 0) ds_part[(size_t)cblock * ld_ds + row] = tot;
}

// FC2 dgrad + dGLU: acc = dA at A columns c0 + ...; gate of A column c sits at
// packed column 64 (c / 32) + c % 32 and the linear value 32 columns further.
// sc: the row's feature scale; ps (in/out): the lane's sum of dA * act.
template <int ACT, class S>
__device__ __forceinline__ void epi_glu_bwd(const S* __restrict__ Hrow, S* __restrict__ Drow,
                                            const f32x16& acc, int c0, int N, float L,
                                            float alpha, int gtanh, float sc, float& ps) {
  float hg[4][4], hl[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    const int pg = (col >> 5) * 64 + (col & 31);
    if (col < N) {
      load4(Hrow + pg, hg[g]);
      load4(Hrow + pg + 32, hl[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    const int pg = (col >> 5) * 64 + (col & 31);
    float dg[4], dl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float gt = hg[g][q], li = hl[g][q], mg = 1.0f, ml = 1.0f;
      if (L > 0.0f) {
        mg = gt <= L ? 1.0f : 0.0f;
        ml = (li >= -L && li <= L) ? 1.0f : 0.0f;
        gt = fminf(gt, L);
        li = fminf(fmaxf(li, -L), L);
      }
      float a, da_dg;
      act_value_grad<ACT>(gt, alpha, gtanh, a, da_dg);
      ps += acc[4 * g + q] * (a * li);
      const float d = acc[4 * g + q] * sc;
      dg[q] = d * li * da_dg * mg;
      dl[q] = d * a * ml;
    }
    store4(Drow + pg, dg);
    store4(Drow + pg + 32, dl);
  }
}

// The same for bf16 H already in registers: hg = {gate, linear} bits of the
// four values at A columns c0 + 8 g .. + 3; dg, dl get their gradients.
template <int ACT>
__device__ __forceinline__ void glu_bwd_raw_group(const u32x2 (&hg)[2], const f32x16& acc, int g,
                                                  float L, float alpha, int gtanh, float sc,
                                                  float& ps, float (&dg)[4], float (&dl)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t wg = hg[0][q >> 1], wl = hg[1][q >> 1];
    float gt = bf16_bits_to_f32((q & 1) ? (wg >> 16) : (wg & 0xffffu));
    float li = bf16_bits_to_f32((q & 1) ? (wl >> 16) : (wl & 0xffffu));
    float mg = 1.0f, ml = 1.0f;
    if (L > 0.0f) {
      mg = gt <= L ? 1.0f : 0.0f;
      ml = (li >= -L && li <= L) ? 1.0f : 0.0f;
      gt = fminf(gt, L);
      li = fminf(fmaxf(li, -L), L);
    }
    float a, da_dg;
    act_value_grad<ACT>(gt, alpha, gtanh, a, da_dg);
    ps += acc[4 * g + q] * (a * li);
    const float d = acc[4 * g + q] * sc;
    dg[q] = d * li * da_dg * mg;
    dl[q] = d * a * ml;
  }
}

template <int ACT>
__device__ __forceinline__ void epi_glu_bwd_raw(const u32x2 (&h)[4][2], uint16_t* __restrict__ Drow,
                                                const f32x16& acc, int c0, int N, float L,
                                                float alpha, int gtanh, float sc, float& ps) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    const int pg = (col >> 5) * 64 + (col & 31);
    float dg[4], dl[4];
    glu_bwd_raw_group<ACT>(h[g], acc, g, L, alpha, gtanh, sc, ps, dg, dl);
    store4(Drow + pg, dg);
    store4(Drow + pg + 32, dl);
  }
}

// FC1 + squared ReLU (not gated): H = acc + b1, A = relu(min(H, L))^2.
template <class S>
__device__ __forceinline__ void epi_srelu_fwd(S* __restrict__ Hrow, S* __restrict__ Arow,
                                              const float* __restrict__ bias, const f32x16& acc,
                                              int c0, int N, float L, float sc) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    float v[4], o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = acc[4 * g + q] + (bias ? bias[col + q] : 0.0f);
      const float h = L > 0.0f ? fminf(v[q], L) : v[q];
      const float r = fmaxf(h, 0.0f);
      o[q] = r * r * sc;
    }
    if (Hrow) store4(Hrow + col, v);
    store4(Arow + col, o);
  }
}

// FC2 dgrad + squared-ReLU backward: dH = dA * 2 relu(h) * [h <= L].
template <class S>
__device__ __forceinline__ void epi_srelu_bwd(const S* __restrict__ Hrow, S* __restrict__ Drow,
                                              const f32x16& acc, int c0, int N, float L, float sc,
                                              float& ps) {
  float hv[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    if (c0 + 8 * g < N) load4(Hrow + c0 + 8 * g, hv[g]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    if (col >= N) continue;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h = hv[g][q], m = 1.0f;
      if (L > 0.0f) {
        m = h <= L ? 1.0f : 0.0f;
        h = fminf(h, L);
      }
      const float r = fmaxf(h, 0.0f);
      ps += acc[4 * g + q] * (r * r);
      o[q] = acc[4 * g + q] * sc * 2.0f * r * m;
    }
    store4(Drow + col, o);
  }
}

// ------------------------------------------------------------------ MXFP8 epilogues
//
// An MXFP8 layer's FC1 and dGLU epilogues write their output (A, dH) as two
// MXFP8 copies quantized from the float32 values: the row copy (blocks of 32
// along the columns, operand of the next forward or dgrad GEMM) and the
// expert-segmented column copy (blocks of 32 along the tokens, operand of the
// weight gradient).  Each 32 x 32 block passes through a wave-private LDS
// tile (row stride 36 floats, so row reads and column reads are both free of
// bank conflicts); lanes 0-31 then quantize one row each, lanes 32-63 one
// column each.

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// The lane's 16 values (columns 8 g + 4 h + q of tile row lane & 31).
__device__ __forceinline__ void mx_stage(float* W, int lane, const float* v) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(W + r * 36 + 8 * g + 4 * h) =
        f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

// Row r0 + l of the row copy gets columns c0 .. c0 + 31 (rows below rlim);
// row c0 + l of the column copy gets token positions p0 .. p0 + 31 (when the
// block starts inside the padded segment, p0 < pend).
// (Element format F: E4M3 blocks take 32 code bytes, E2M1 blocks 16.)
template <class F>
__device__ __forceinline__ void mx_store_block(uint8_t* dst, const uint32_t* w) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  d[0] = u32x4{w[0], w[1], w[2], w[3]};
  if constexpr (F::WORDS == 8) d[1] = u32x4{w[4], w[5], w[6], w[7]};
}

template <class F = FmtE4M3>
__device__ __forceinline__ void mx_emit(const float* W, int lane, const GemmArgs& p, int r0,
                                        int rlim, int c0, int p0, int pend) {
  constexpr int B = F::BYTES;
  const int l = lane & 31;
  float v[32];
  uint32_t w8[8];
  if (lane < 32) {
    const int row = r0 + l;
    if (p.mxr && row < rlim) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(W + l * 36 + 4 * q);
        v[4 * q] = t[0];
        v[4 * q + 1] = t[1];
        v[4 * q + 2] = t[2];
        v[4 * q + 3] = t[3];
      }
      const uint32_t sc = mx_quant32<F>(v, w8);
      mx_store_block<F>(p.mxr + (size_t)row * (p.ld_mxr / 32 * B) + c0 / 32 * B, w8);
      p.mxr_s[(size_t)row * (p.ld_mxr / 32) + c0 / 32] = (uint8_t)sc;
    }
  } else if (p.mxc && p0 < pend) {
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = W[r * 36 + l];
    const uint32_t sc = mx_quant32<F>(v, w8);
    mx_store_block<F>(p.mxc + (size_t)(c0 + l) * (p.ld_mxc / 32 * B) + p0 / 32 * B, w8);
    p.mxc_s[(size_t)(c0 + l) * (p.ld_mxc / 32) + p0 / 32] = (uint8_t)sc;
  }
}

// The same for two staged 32 x 32 blocks at once: block 1 (W1) at rows r1,
// columns c1, token positions p1 .. p1 + 31, block 2 (W2) at r2, c2, p2.
// Lanes 0-31 quantize block 1's rows and then its columns, lanes 32-63 block
// 2's, so every lane runs the same instructions (one block at a time splits
// the wave into a row half and a column half, each running the whole
// quantizer with the other half masked off).
template <class F = FmtE4M3>
__device__ __forceinline__ void mx_emit_two(const float* W1, const float* W2, int lane,
                                            const GemmArgs& p, int r1, int r2, int c1, int c2,
                                            int p1, int p2, int rlim, int pend) {
  constexpr int B = F::BYTES;
  const int l = lane & 31;
  const bool two = lane >= 32;
  const float* W = two ? W2 : W1;
  const int r0 = two ? r2 : r1, cb = two ? c2 : c1, p0 = two ? p2 : p1;
  float v[32];
  uint32_t w8[8];
  const int row = r0 + l;
  if (p.mxr && row < rlim) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(W + l * 36 + 4 * q);
      v[4 * q] = t[0];
      v[4 * q + 1] = t[1];
      v[4 * q + 2] = t[2];
      v[4 * q + 3] = t[3];
    }
    const uint32_t sc = mx_quant32<F>(v, w8);
    mx_store_block<F>(p.mxr + (size_t)row * (p.ld_mxr / 32 * B) + cb / 32 * B, w8);
    p.mxr_s[(size_t)row * (p.ld_mxr / 32) + cb / 32] = (uint8_t)sc;
  }
  if (p.mxc && p0 < pend) {
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = W[r * 36 + l];
    const uint32_t sc = mx_quant32<F>(v, w8);
    mx_store_block<F>(p.mxc + (size_t)(cb + l) * (p.ld_mxc / 32 * B) + p0 / 32 * B, w8);
    p.mxc_s[(size_t)(cb + l) * (p.ld_mxc / 32) + p0 / 32] = (uint8_t)sc;
  }
}

// FC1 + GLU values of one gate/linear block pair: stores H (bf16, nullable
// row pointer), returns A (zero for rows past the segment).
template <int ACT>
__device__ __forceinline__ void glu_fwd_values(uint16_t* __restrict__ Hrow, const f32x16& accg,
                                               const f32x16& accl, int c0, float L, float alpha,
                                               int gtanh, bool rok, float sc, float* o) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    float gv[4], lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gv[q] = accg[4 * g + q];
      lv[q] = accl[4 * g + q];
    }
    if (Hrow) {
      store4(Hrow + col, gv);
      store4(Hrow + col + 32, lv);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float gt = gv[q], li = lv[q];
      if (L > 0.0f) {
        gt = fminf(gt, L);
        li = fminf(fmaxf(li, -L), L);
      }
      o[4 * g + q] = rok ? act_value<ACT>(gt, alpha, gtanh) * li * sc : 0.0f;
    }
  }
}

// The saved H values one lane needs for a 32 x 32 block of dA whose first
// column (of this lane) is c0: gate and linear bf16 of 4 runs of 4 columns,
// as raw bits (zeros when Hrow is NULL, i.e. the row is past the segment).
__device__ __forceinline__ void glu_bwd_hload(const uint16_t* __restrict__ Hrow, int c0,
                                              u32x2 (&h)[4][2]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = c0 + 8 * g;
    const int pg = (col >> 5) * 64 + (col & 31);
    h[g][0] = Hrow ? *reinterpret_cast<const u32x2*>(Hrow + pg) : u32x2{0u, 0u};
    h[g][1] = Hrow ? *reinterpret_cast<const u32x2*>(Hrow + pg + 32) : u32x2{0u, 0u};
  }
}

// dGLU of one block from its loaded H (glu_bwd_hload); `live` = the row is
// inside the segment (else the outputs are 0).
template <int ACT>
__device__ __forceinline__ void glu_bwd_values_h(const u32x2 (&h)[4][2], bool live,
                                                 const f32x16& acc, float L, float alpha,
                                                 int gtanh, float sc, float& ps, float* dg,
                                                 float* dl) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float hg[4], hl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hg[q] = bf16_bits_to_f32((h[g][0][q >> 1] >> (16 * (q & 1))) & 0xffffu);
      hl[q] = bf16_bits_to_f32((h[g][1][q >> 1] >> (16 * (q & 1))) & 0xffffu);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float gt = hg[q], li = hl[q], mg = 1.0f, ml = 1.0f;
      if (L > 0.0f) {
        mg = gt <= L ? 1.0f : 0.0f;
        ml = (li >= -L && li <= L) ? 1.0f : 0.0f;
        gt = fminf(gt, L);
        li = fminf(fmaxf(li, -L), L);
      }
      float a, da_dg;
      act_value_grad<ACT>(gt, alpha, gtanh, a, da_dg);
      const float dr = live ? acc[4 * g + q] : 0.0f;
      ps += dr * (a * li);
      const float d = dr * sc;
      dg[4 * g + q] = d * li * da_dg * mg;
      dl[4 * g + q] = d * a * ml;
    }
  }
}

// Workgroup barrier for the LDS ring.  __syncthreads() (and any fence whose
// scope covers LDS) makes the compiler wait for every outstanding load first,
// including the LDS-DMA loads of later ring stages, which would serialise the
// pipeline.  Here each wave has already waited (vm_wait) for its loads into
// the stage about to be read, and its reads of the stage about to be
// overwritten have been consumed by MFMAs, so a bare s_barrier suffices; the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until this wave's LDS reads have returned.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(N): wait until at most N vector-memory loads of this wave are
// outstanding (expcnt and lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` whole steps (PERW loads each) are still in flight.
template <int PERW, int MAXAHEAD>
__device__ __forceinline__ void vm_wait_steps(int ahead) {
  static_assert(MAXAHEAD <= 3 && 3 * PERW <= 63, "vmcnt holds at most 63");
  if constexpr (MAXAHEAD >= 3) {
    if (ahead >= 3) {
      vm_wait<3 * PERW>();
      return;
    }
  }
  if constexpr (MAXAHEAD >= 2) {
    if (ahead >= 2) {
      vm_wait<2 * PERW>();
      return;
    }
  }
  if constexpr (MAXAHEAD >= 1) {
    if (ahead >= 1) {
      vm_wait<PERW>();
      return;
    }
  }
  vm_wait<0>();
}

// ------------------------------------------------------------------ the kernel

// Tile policy: block tile BM x BN, WGM x WGN waves, BKB bytes of K per pipeline
// step, STAGES-deep LDS ring.
// SCHED = 1 pins the k-step's instruction order: the first sub-step's fragment
// reads, then one MFMA at a time with the next sub-step's reads spread between.
template <int BM_, int BN_, int WGM_, int WGN_, int BKB_, int STAGES_, int SCHED_ = 0>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BKB = BKB_, STAGES = STAGES_;
  static constexpr int SCHED = SCHED_;
};

template <class EL, int EPI, class TL>
struct GemmCfg {
  static constexpr int BM = TL::BM, BN = TL::BN, WGM = TL::WGM, WGN = TL::WGN;
  static constexpr int THREADS = WGM * WGN * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int BKB = TL::BKB;
  static constexpr int BK = BKB / sizeof(typename EL::storage);   // k per pipeline step
  static constexpr bool MX = is_mx<EL>();
  static constexpr int EPB = epb<EL>();                            // k elements per byte
  static constexpr int SUB = MX ? BKB * EPB / 64 : BKB / 32;       // MFMA k sub-steps per step
  static constexpr int STAGES = TL::STAGES;                        // LDS ring depth
  // 16-byte units per stage: the A and B tiles, then (MX) one scale word per row
  static constexpr int STAGE_U4 = (BM + BN) * (BKB / 16) + (MX ? (BM + BN) / 4 : 0);
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_U4 * 16;
  // MX epilogues stage 32 x 36 floats per wave in the ring slots that are
  // free after the main loop: STAGE_WAVES waves per slot, MX_SLOTS slots
  static constexpr int MX_STAGE_FLOATS = 32 * 36;
  static constexpr int STAGE_WAVES = STAGE_U4 * 16 / (MX_STAGE_FLOATS * 4);
  static constexpr int MX_SLOTS = (THREADS / 64 + STAGE_WAVES - 1) / STAGE_WAVES;
  // The plain epilogue can stage 32 rows of each wave's tile (in the output
  // type OT) in the ring slots free after the main loop before writing whole
  // rows, where every wave's rows fit in them.
  template <class OT>
  static constexpr bool stage_fits() {
    return stage_waves<OT>() >= 1 &&
           (THREADS / 64 + stage_waves<OT>() - 1) / stage_waves<OT>() <= STAGES - 1 &&
           (WTN * (int)sizeof(OT) == 128 || WTN * (int)sizeof(OT) == 256);
  }
  // waves whose 32-row staging tiles fit one ring slot (the staged plain
  // epilogue spreads the waves over the STAGES - 1 slots free after the main
  // loop)
  template <class OT>
  static constexpr int stage_waves() {
    return STAGE_U4 * 16 / (32 * WTN * (int)sizeof(OT));
  }
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!epi_glu_fwd(EPI) || WTN % 64 == 0, "GLU pairs need 64-column wave tiles");
  static_assert(LDS_BYTES + 8320 <= 160 * 1024, "LDS ring does not fit");
  static_assert(!MX || (STAGE_WAVES >= 1 && MX_SLOTS <= STAGES - 1),
                "MX epilogue staging must fit in the free ring slots");
  static_assert(!MX || BKB * EPB == 128, "MX steps are 128 k (four scale blocks, one word)");
};

// RS: the feature-scaling variant of a GLU / sReLU epilogue (row_scale,
// ds_part); without it those fields are ignored and the code is the plain one.
template <class EL, bool AKM, bool BKM, int GROUP, int EPI, class TL, bool GATHER = false,
          bool RS = false>
__global__ void __launch_bounds__(TL::WGM * TL::WGN * 64)
    grouped_gemm_kernel(GemmArgs p) {
  typedef GemmCfg<EL, EPI, TL> C;
  constexpr int BM = C::BM, BN = C::BN, WGN = C::WGN;
  typedef typename EL::storage S;
  constexpr int THREADS = C::THREADS, TM = C::TM, TN = C::TN, BK = C::BK;
  extern __shared__ u32x4 smem[];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_tab[MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int E = p.E;

  // ---- tile table (device-side shapes) ----
  for (int e = tid; e <= E; e += THREADS) {
    int o = p.offsets[e];
    o = o < 0 ? 0 : (o > p.R ? p.R : o);
    // K counts bytes: MXFP4 weight-gradient segments (32-element aligned) halve
    s_off[e] = GROUP == RAGGED_K ? o / epb<EL>() : o;
  }
  __syncthreads();
  int total;
  int mt_k = 0, nt_k = 0;
  const int nN = (p.N + BN - 1) / BN;
  if constexpr (GROUP == RAGGED_M) {
    // s_tab[e] = exclusive prefix of the M-tiles of experts < e (wave 0 scans)
    if (wave == 0) {
      constexpr int PER = (MOE_MAX_EXPERTS + 63) / 64;
      int sum = 0;
      for (int i = 0; i < PER; ++i) {
        int e = lane * PER + i;
        if (e < E) sum += (max(s_off[e + 1] - s_off[e], 0) + BM - 1) / BM;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      int run = incl - sum;
      for (int i = 0; i < PER; ++i) {
        int e = lane * PER + i;
        if (e < E) {
          s_tab[e] = run;
          run += (max(s_off[e + 1] - s_off[e], 0) + BM - 1) / BM;
        }
      }
      if (lane == 63) s_tab[E] = incl;
    }
    __syncthreads();
    total = s_tab[E] * nN;
  } else {
    // s_tab[rank] = expert, by decreasing row count (ties: lower id first)
    for (int e = tid; e < E; e += THREADS) {
      int ce = max(s_off[e + 1] - s_off[e], 0), rank = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        int c2 = max(s_off[e2 + 1] - s_off[e2], 0);
        rank += (c2 > ce) || (c2 == ce && e2 < e);
      }
      s_tab[rank] = e;
    }
    __syncthreads();
    mt_k = (p.M + BM - 1) / BM;
    nt_k = nN;
    total = E * mt_k * nt_k;
  }

  const int G = gridDim.x;
  const int vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // ---- tile decode: expert, row / column origin, row limit, k range ----
  struct TileC {
    int e, m0, n0, mlim, kbeg, kend;
    int kb0;  // first k of the first step (MX weight gradients: kbeg rounded down to a step)
  };
  auto decode = [&](int tile) {
    TileC t;
    if constexpr (GROUP == RAGGED_M) {
      const int total_m = s_tab[E];
      const int span = p.gm * nN;
      int band = tile / span, in = tile - band * span;
      int first = band * p.gm;
      int gsz = min(total_m - first, p.gm);
      int gm = first + in % gsz;
      int nt = in / gsz;
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (s_tab[mid] <= gm) lo = mid; else hi = mid;
      }
      t.e = lo;
      t.m0 = s_off[lo] + (gm - s_tab[lo]) * BM;
      t.mlim = s_off[lo + 1];
      t.n0 = nt * BN;
      t.kbeg = 0;
      t.kend = p.K;
    } else {
      const int per = mt_k * nt_k;
      int slot = tile / per, in = tile - slot * per;
      t.e = s_tab[slot];
      const int span = p.gm_k * nt_k;
      int band = in / span, r = in - band * span;
      int first = band * p.gm_k;
      int gsz = min(mt_k - first, p.gm_k);
      t.m0 = (first + r % gsz) * BM;
      t.n0 = (r / gsz) * BN;
      t.mlim = p.M;
      t.kbeg = s_off[t.e];
      t.kend = max(s_off[t.e + 1], t.kbeg);
    }
    // The coordinates come out of LDS tables but are the same on every lane:
    // say so, so that addresses and buffer descriptors live in SGPRs.
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.mlim = __builtin_amdgcn_readfirstlane(t.mlim);
    t.kbeg = __builtin_amdgcn_readfirstlane(t.kbeg);
    t.kend = __builtin_amdgcn_readfirstlane(t.kend);
    t.kb0 = (C::MX && GROUP == RAGGED_K) ? (t.kbeg & ~(BK - 1)) : t.kbeg;
    return t;
  };

  // Both operands go global -> LDS by DMA into a ring of STAGES buffers.
  // Step kt waits until its own buffer has landed while the loads of the next
  // STAGES - 2 steps stay in flight, meets the other waves at a barrier (after
  // which nobody reads the buffer of step kt - 1 any more), refills that
  // buffer with step kt + STAGES - 1, and runs the MFMAs of step kt.  (Issuing
  // the next tile's first loads before the epilogue was measured: it gains
  // nothing, and the ring position it needs costs more than that.)
  constexpr int BKB = C::BKB, SUB = C::SUB, CPR = BKB / 16;
  // the gathered operand: A's rows (RAGGED_M) or B's k-rows (RAGGED_K)
  constexpr bool GA = GATHER && GROUP == RAGGED_M, GB = GATHER && GROUP == RAGGED_K;
  static_assert(!GATHER || (GA ? AKM : !BKM), "gathers whole K-rows or whole k-rows");
  typedef typename std::conditional<AKM, DmaK<EL, BM, THREADS, BKB, GA>,
                                    DmaMN<EL, BM, THREADS, BKB, GA>>::type LoadA;
  typedef typename std::conditional<BKM, DmaK<EL, BN, THREADS, BKB, GB>,
                                    DmaMN<EL, BN, THREADS, BKB, GB>>::type LoadB;
  constexpr int S_ = C::STAGES;
  constexpr bool MX = C::MX;
  static_assert(!MX || (AKM && BKM), "MXFP8 operands are K-contiguous");
  // DMA instructions per wave per step (MX: plus one scale word load)
  constexpr int PERW = LoadA::PER + LoadB::PER + (MX ? 1 : 0);
  struct NoScale {};
  typename std::conditional<MX, DmaScale<BM, BN, THREADS>, NoScale>::type ls;
  auto scales_of = [&](const u32x4* st) {
    return reinterpret_cast<uint32_t*>(const_cast<u32x4*>(st) + (BM + BN) * CPR);
  };
  const S* A = reinterpret_cast<const S*>(p.a);
  LoadA la;
  LoadB lb;
  auto stage_ptr = [&](int st) { return smem + (st % S_) * C::STAGE_U4; };
  auto nk_of = [&](const TileC& t) {
    return t.kend > t.kbeg ? (t.kend - t.kb0 + BK - 1) / BK : 0;
  };
  // set the loaders up for tile t and issue its first STAGES - 1 steps
  auto prologue = [&](const TileC& t) {
    const S* B = reinterpret_cast<const S*>(p.b);
    if constexpr (GROUP == RAGGED_M) B += (size_t)t.e * p.b_expert_stride;
    if constexpr (GROUP == RAGGED_M) {
      la.setup(A, p.lda, t.m0, t.mlim, t.kend, tid, t.kbeg, p.gather, p.gather_rows);
      lb.setup(B, p.ldb, t.n0, p.N, t.kend, tid, t.kbeg);
    } else {
      la.setup(A, p.lda, t.m0, t.mlim, t.kend, tid, t.kbeg);
      lb.setup(B, p.ldb, t.n0, p.N, t.kend, tid, t.kbeg, p.gather, p.gather_rows);
    }
    if constexpr (MX) {
      const uint8_t* SB = p.sb;
      if constexpr (GROUP == RAGGED_M) SB += (size_t)t.e * p.sb_expert_stride;
      ls.setup(p.sa, p.slda, t.m0, t.mlim, SB, p.sldb, t.n0, p.N, tid);
    }
    const int nk = nk_of(t);
#pragma unroll
    for (int st = 0; st < S_ - 1; ++st)
      if (st < nk) {
        la.issue(stage_ptr(st), t.kb0 + st * BK);
        lb.issue(stage_ptr(st) + BM * CPR, t.kb0 + st * BK);
        if constexpr (MX) ls.issue(scales_of(stage_ptr(st)), (t.kb0 + st * BK) * C::EPB);
      }
  };

  // Round r gives block vb the tile r G + vb.  Weight-gradient tiles are
  // ordered by decreasing k length (experts largest first), so there odd
  // rounds run backwards (r G + G - 1 - vb): a block that took one of the
  // longest tiles of a round takes one of the shortest of the next, which
  // evens out the per-block sums.  Either way the 32 blocks of an XCD take 32
  // consecutive tiles of a round.
  for (int round = 0;; ++round) {
    const int tile = round * G + ((GROUP == RAGGED_K && p.snake && (round & 1)) ? G - 1 - vb : vb);
    if (tile >= total) break;
    const TileC cur = decode(tile);
    const int nk = nk_of(cur);
    __syncthreads();  // every wave is done with the previous tile's buffers
    prologue(cur);

    // ---- main loop ----
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if constexpr (TL::SCHED == 2) {
      // Ping-pong: wave group g (= wm, one wave per SIMD) alternates a memory
      // phase (read every fragment of one k-step into registers) and a
      // compute phase (that step's MFMAs from registers), the two groups one
      // phase apart, so that on each SIMD one wave is always feeding the MFMA
      // pipe.  Phase t: group 0 reads step t / 2 (t even) and computes step
      // (t - 1) / 2 (t odd); group 1 one phase later.  Every wave ends every
      // phase at a barrier, after its LDS reads have returned.  Both groups
      // have read step j by the end of phase 2 j + 1, so step j + S is loaded
      // into step j's slot at the start of phase 2 j + 2; the loads of step
      // j + 1 are waited for at the end of phase 2 j + 1.
      // (with 4 wave rows, rows 0 and 2 form group 0 and rows 1 and 3 group 1:
      // each SIMD then holds two waves of each group)
      static_assert(C::WGM % 2 == 0 && !MX, "ping-pong needs two wave groups");
      const int grp = wm & 1;
#pragma unroll
      for (int st = S_ - 1; st < S_; ++st)
        if (st < nk) {
          la.issue(stage_ptr(st), cur.kb0 + st * BK);
          lb.issue(stage_ptr(st) + BM * CPR, cur.kb0 + st * BK);
        }
      // step 0 landed; the loads of steps 1 .. min(S, nk) - 1 may still fly
      vm_wait_steps<PERW, S_ - 1>(min(S_, nk) - 1);
      lds_barrier();
      u32x4 fa[SUB][TM], fb[SUB][TN];
      auto mem = [&](int j) {  // every fragment of step j into registers
        const u32x4* As = stage_ptr(j);
        const u32x4* Bs = As + BM * CPR;
#pragma unroll
        for (int s2 = 0; s2 < SUB; ++s2) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
            fa[s2][i] = Frag<AKM, EL, BM, BKB>::load(As, wm * C::WTM + 32 * i, s2, lane);
#pragma unroll
          for (int jj = 0; jj < TN; ++jj)
            fb[s2][jj] = Frag<BKM, EL, BN, BKB>::load(Bs, wn * C::WTN + 32 * jj, s2, lane);
        }
      };
      auto comp = [&]() {      // that step's MFMAs
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < SUB; ++s2)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) mma(acc[i][jj], fb[s2][jj], fa[s2][i], EL());
        __builtin_amdgcn_s_setprio(0);
      };
      auto end_even = [&]() {  // end of phase 2 j (or 2 j + 2)
        lds_wait();
        lds_barrier();
      };
      auto end_odd = [&](int j) {  // end of phase 2 j + 1
        lds_wait();
        // step j + 1 must have landed; steps up to j + S - 1 may still fly
        vm_wait_steps<PERW, S_ - 2>(min(S_ - 2, nk - 2 - j));
        lds_barrier();
        if (j + S_ < nk) {  // both groups have read step j: refill its slot
          u32x4* nb = stage_ptr(j + S_);
          la.issue(nb, cur.kb0 + (j + S_) * BK);
          lb.issue(nb + BM * CPR, cur.kb0 + (j + S_) * BK);
        }
      };
      // group 0: read step j in phase 2 j, compute it in 2 j + 1; group 1 one
      // phase later.  Both pass the same 2 nk + 1 barriers.
      if (grp == 0) {
        for (int j = 0; j < nk; ++j) {
          mem(j);
          end_even();
          comp();
          end_odd(j);
        }
        end_even();
      } else {
        end_even();
        for (int j = 0; j < nk; ++j) {
          mem(j);
          end_odd(j);
          comp();
          end_even();
        }
      }
    } else
    for (int kt = 0; kt < nk; ++kt) {
      // loads issued after step kt's: steps kt+1 .. min(kt+S-2, nk-1)
      vm_wait_steps<PERW, S_ - 2>(min(S_ - 2, nk - 1 - kt));
      lds_barrier();
      if (kt + S_ - 1 < nk) {
        u32x4* nb = stage_ptr(kt + S_ - 1);
        la.issue(nb, cur.kb0 + (kt + S_ - 1) * BK);
        lb.issue(nb + BM * CPR, cur.kb0 + (kt + S_ - 1) * BK);
        if constexpr (MX) ls.issue(scales_of(nb), (cur.kb0 + (kt + S_ - 1) * BK) * C::EPB);
      }
      const u32x4* As = stage_ptr(kt);
      const u32x4* Bs = As + BM * CPR;
      if constexpr (MX) {
        // scale word of each fragment row, shifted so that byte 2 s holds the
        // block of sub-step s that this lane's half (h) covers: 2 s + h
        const int h = lane >> 5;
        const uint32_t* Ss = scales_of(As);
        uint32_t swa[TM], swb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) swa[i] = Ss[wm * C::WTM + 32 * i + (lane & 31)] >> (8 * h);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          swb[j] = Ss[BM + wn * C::WTN + 32 * j + (lane & 31)] >> (8 * h);
        if constexpr (GROUP == RAGGED_K) {
          // blocks outside the segment read zero codes; their scale bytes
          // belong to other segments (or were never written): make them 1.0
          const int b0 = (cur.kb0 + kt * BK) * C::EPB / 32 + h;
          uint32_t keep = 0xffffffffu, fill = 0u;
#pragma unroll
          for (int s2 = 0; s2 < SUB; ++s2) {
            const int b = b0 + 2 * s2;
            if (b * 32 < cur.kbeg * C::EPB || b * 32 >= cur.kend * C::EPB) {
              keep &= ~(0xffu << (16 * s2));
              fill |= 127u << (16 * s2);
            }
          }
#pragma unroll
          for (int i = 0; i < TM; ++i) swa[i] = (swa[i] & keep) | fill;
#pragma unroll
          for (int j = 0; j < TN; ++j) swb[j] = (swb[j] & keep) | fill;
        }
        u32x8 af[2][TM], bfr[2][TN];
        auto frags = [&](int buf, int s2) {
          af[buf][0] = FragMX<BM, BKB, EL>::load(As, wm * C::WTM, s2, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            bfr[buf][j] = FragMX<BN, BKB, EL>::load(Bs, wn * C::WTN + 32 * j, s2, lane);
#pragma unroll
          for (int i = 1; i < TM; ++i)
            af[buf][i] = FragMX<BM, BKB, EL>::load(As, wm * C::WTM + 32 * i, s2, lane);
        };
        frags(0, 0);
        static_for<0, SUB>([&](auto sc) {
          constexpr int s2 = decltype(sc)::value;
          if constexpr (s2 + 1 < SUB) frags((s2 + 1) & 1, s2 + 1);
          static_for<0, TM>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<0, TN>([&](auto jc) {
              constexpr int j = decltype(jc)::value;
              mma_mx<2 * s2, EL::FMT>(acc[i][j], bfr[s2 & 1][j], af[s2 & 1][i], swb[j],
                                      swa[i]);
            });
          });
        });
        if constexpr (TL::SCHED == 1) {
          constexpr int NR = (TM + TN) * FragMX<BM, BKB, EL>::READS;
          constexpr int NM = TM * TN;
          __builtin_amdgcn_sched_group_barrier(0x100, NR + TM + TN, 0);
          static_for<0, SUB>([&](auto s2) {
            static_for<0, NM>([&](auto m) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              constexpr int nr = (NR * (m + 1)) / NM - (NR * m) / NM;
              if constexpr (s2 + 1 < SUB && nr > 0)
                __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
            });
          });
        }
      } else {
        // fragments of sub-step s + 1 are read while the MFMAs of s run;
        // read in order of first use by the i-major MFMA loop: a0, b0 .. b(TN-1), a1 ..
        u32x4 af[2][TM], bfr[2][TN];
        auto frags = [&](int buf, int s2) {
          af[buf][0] = Frag<AKM, EL, BM, BKB>::load(As, wm * C::WTM, s2, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            bfr[buf][j] = Frag<BKM, EL, BN, BKB>::load(Bs, wn * C::WTN + 32 * j, s2, lane);
#pragma unroll
          for (int i = 1; i < TM; ++i)
            af[buf][i] = Frag<AKM, EL, BM, BKB>::load(As, wm * C::WTM + 32 * i, s2, lane);
        };
        frags(0, 0);
#pragma unroll
        for (int s2 = 0; s2 < SUB; ++s2) {
          if (s2 + 1 < SUB) frags((s2 + 1) & 1, s2 + 1);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) mma(acc[i][j], bfr[s2 & 1][j], af[s2 & 1][i], EL());
        }
        if constexpr (TL::SCHED == 1) {
          constexpr int NR = TM * Frag<AKM, EL, BM, BKB>::READS + TN * Frag<BKM, EL, BN, BKB>::READS;
          constexpr int NM = TM * TN;
          __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
          static_for<0, SUB>([&](auto s2) {
            static_for<0, NM>([&](auto m) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              constexpr int nr = (NR * (m + 1)) / NM - (NR * m) / NM;
              if constexpr (s2 + 1 < SUB && nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
            });
          });
        }
      }  // bf16 / fp32 step
    }
    const int e = cur.e, m0 = cur.m0, n0 = cur.n0, mlim = cur.mlim;

    // ---- epilogue: lane holds rows (lane & 31) + 32 i, columns 32 j + 8 g + 4 h + q ----
    typedef typename OutT<EL>::type SO;
    const int cw = n0 + wn * C::WTN + 4 * (lane >> 5);  // column of the lane's first value
    // output element of the plain epilogue: the storage type (RAGGED_M) or
    // float32 (weight gradients)
    typedef typename std::conditional<GROUP == RAGGED_M, SO, float>::type OT;
    // (built where it needs no spills: the plain bf16 epilogue of tiles with
    // both operands K-contiguous and the pinned or compiler schedule -- FC2
    // and the FC1 dgrad from the transposed weights -- whose direct stores
    // wrote 1.58x the output bytes; and the weight gradients' float32 stores,
    // which already wrote 1.03-1.08x but cost 9 % of those kernels as
    // 32-byte pieces of 32 rows per store, 3 % less as whole rows)
    constexpr bool kStaged = EPI == EPI_STORE && (!MX || GROUP == RAGGED_K) &&
                             (GROUP == RAGGED_K || (AKM && BKM && TL::SCHED != 2)) &&
                             C::template stage_fits<OT>();
    // FC1 + GLU (bf16, 64-column wave tiles): H and A through LDS the same way
    constexpr bool kStagedGlu = epi_glu_fwd(EPI) && GROUP == RAGGED_M && !MX &&
                                TL::SCHED != 2 && sizeof(SO) == 2 && C::WTN == 64 &&
                                (THREADS / 64) * 32 * (C::WTN * 2 + C::WTN) <= C::STAGE_U4 * 16;
    // FC2 dgrad + dGLU (bf16, 64-column wave tiles, no feature-scaling
    // gradient: with it the kernel spills): dH through LDS as 256-byte rows
    constexpr bool kStagedDglu = epi_glu_bwd(EPI) && GROUP == RAGGED_M && !MX && !RS &&
                                 TL::SCHED != 2 && sizeof(SO) == 2 && C::WTN == 64 &&
                                 (THREADS / 64) * 32 * (C::WTN * 2 * 2) <= C::STAGE_U4 * 16;
#ifdef MOE_GEMM_TUNING
    const bool glu_direct = p.glu_direct == 1, glu_a_direct = p.glu_direct == 2;
#else
    constexpr bool glu_direct = false, glu_a_direct = false;
#endif
    bool mx_store = false;  // plain product written as an MX row copy instead of C
    if constexpr (MX && EPI == EPI_STORE && GROUP == RAGGED_M) mx_store = p.mxr != nullptr;
    if (mx_store) {
      if constexpr (MX && EPI == EPI_STORE && GROUP == RAGGED_M) {
        // the 32 x 32 blocks of column blocks j and j + 1 pass through two
        // staging tiles of the wave together; lanes 0-31 quantize one row
        // each of the first, lanes 32-63 of the second (blocks of 32
        // columns).  The second tiles may reach into the last step's ring
        // slot, which all waves have finished reading past this barrier.
        constexpr int NW = THREADS / 64;
        static_assert(2 * NW <= C::STAGES * C::STAGE_WAVES && TN % 2 == 0,
                      "two staging areas per wave");
        __syncthreads();
        float* Wt = reinterpret_cast<float*>(stage_ptr(nk + wave / C::STAGE_WAVES)) +
                    (wave % C::STAGE_WAVES) * C::MX_STAGE_FLOATS;
        float* Wt2 = reinterpret_cast<float*>(stage_ptr(nk + (NW + wave) / C::STAGE_WAVES)) +
                     ((NW + wave) % C::STAGE_WAVES) * C::MX_STAGE_FLOATS;
        static_for<0, TM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const int r0 = m0 + wm * C::WTM + 32 * i;
          static_for<0, TN / 2>([&](auto jc) {
            constexpr int j = 2 * decltype(jc)::value;
            const int cb = n0 + wn * C::WTN + 32 * j;
            if (cb < p.N) {
              float o[16];
#pragma unroll
              for (int r = 0; r < 16; ++r) o[r] = acc[i][j][r];
              mx_stage(Wt, lane, o);
#pragma unroll
              for (int r = 0; r < 16; ++r) o[r] = acc[i][j + 1][r];
              mx_stage(Wt2, lane, o);
              wave_lds_sync();
              // a second block past N writes nothing: its rows start at mlim
              mx_emit_two<typename EL::Fmt>(Wt, Wt2, lane, p, r0, cb + 32 < p.N ? r0 : mlim, cb,
                                            cb + 32, 0, 0, mlim, 0);
              wave_lds_sync();
            }
          });
        });
      }
    } else if constexpr (MX && (epi_glu_fwd(EPI) || epi_glu_bwd(EPI))) {
      // every lane takes part (the tile is shared); rows past the segment are
      // zero in the column copy and skipped in the row copy.  The ring slot
      // after the last step's is free: its last reader passed the barrier of
      // the last step, and the next tile's loads start after a barrier.
      float* Wt = reinterpret_cast<float*>(stage_ptr(nk + wave / C::STAGE_WAVES)) +
                  (wave % C::STAGE_WAVES) * C::MX_STAGE_FLOATS;
      // Two blocks are staged and quantized together (dGLU: the gate and the
      // linear block of a column block; GLU forward: the A blocks of row
      // blocks 2 h and 2 h + 1).  The second takes the next staging areas,
      // which may reach into the last step's ring slot: every wave has
      // finished reading it once all have passed the barrier below, and no
      // load is in flight after the last step.  For the GLU forward only
      // with E4M3 codes: with E2M1 the pairing measured 21 % slower there
      // (and 4 % faster for the dGLU).
      constexpr bool kPair = epi_glu_bwd(EPI) || EL::Fmt::WORDS == 8;
      float* Wt2 = nullptr;
      if constexpr (kPair) {
        constexpr int NW = THREADS / 64;
        static_assert(2 * NW <= C::STAGES * C::STAGE_WAVES, "two staging areas per wave");
        __syncthreads();
        Wt2 = reinterpret_cast<float*>(stage_ptr(nk + (NW + wave) / C::STAGE_WAVES)) +
              ((NW + wave) % C::STAGE_WAVES) * C::MX_STAGE_FLOATS;
      }
      const int pe0 = p.pad_offsets ? p.pad_offsets[e] : 0;
      const int pe1 = p.pad_offsets ? p.pad_offsets[e + 1] : 0;
      const int off_e = s_off[e];
      u32x2 hbuf[2][4][2];  // dGLU: saved H of the current and the next block
      if constexpr (epi_glu_bwd(EPI)) {
        const int row0 = m0 + wm * C::WTM + (lane & 31);
        const int cb0 = n0 + wn * C::WTN;
        glu_bwd_hload((row0 < mlim && cb0 < p.N)
                          ? reinterpret_cast<const SO*>(p.aux) + (size_t)row0 * p.ld_aux
                          : nullptr,
                      cb0 + 4 * (lane >> 5), hbuf[0]);
      }
      static_for<0, TM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int r0 = m0 + wm * C::WTM + 32 * i;
        const int row = r0 + (lane & 31);
        const bool rok = row < mlim;
        const int prow = pe0 + (r0 - off_e);
        const float sc = (RS && rok && p.row_scale) ? p.row_scale[row] : 1.0f;
        static_for<0, TN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int cb = n0 + wn * C::WTN + 32 * j;
          if constexpr (epi_glu_fwd(EPI)) {
            if constexpr ((j & 1) == 0) {
              if (cb < p.N) {
                float o[16];
                glu_fwd_values<epi_act(EPI)>(
                    (rok && p.aux) ? reinterpret_cast<SO*>(p.aux) + (size_t)row * p.ld_aux
                                   : nullptr,
                    acc[i][j], acc[i][j + 1], cb + 4 * (lane >> 5), p.clamp, p.alpha,
                    p.gelu_tanh, rok, sc, o);
                const int ca = (cb >> 6) * 32;
                // row blocks 2 h and 2 h + 1 go out together
                mx_stage((kPair && (i & 1)) ? Wt2 : Wt, lane, o);
                if constexpr (!kPair) {
                  wave_lds_sync();
                  mx_emit<typename EL::Fmt>(Wt, lane, p, r0, mlim, ca, prow, pe1);
                  wave_lds_sync();
                } else if constexpr ((i & 1) == 1) {
                  wave_lds_sync();
                  mx_emit_two<typename EL::Fmt>(Wt, Wt2, lane, p, r0 - 32, r0, ca, ca,
                                                prow - 32, prow, mlim, pe1);
                  wave_lds_sync();
                } else if constexpr (i + 1 == TM) {
                  wave_lds_sync();
                  mx_emit<typename EL::Fmt>(Wt, lane, p, r0, mlim, ca, prow, pe1);
                  wave_lds_sync();
                }
              }
            }
          } else {
            // the saved H of the next block (j + 1, or row block i + 1) is
            // requested before this block is computed and stored, so its load
            // latency hides behind this block's quantization
            constexpr int b = i * TN + j;
            if constexpr (b + 1 < TM * TN) {
              constexpr int i2 = (b + 1) / TN, j2 = (b + 1) % TN;
              const int row2 = m0 + wm * C::WTM + 32 * i2 + (lane & 31);
              const int cb2 = n0 + wn * C::WTN + 32 * j2;
              glu_bwd_hload((row2 < mlim && cb2 < p.N)
                                ? reinterpret_cast<const SO*>(p.aux) + (size_t)row2 * p.ld_aux
                                : nullptr,
                            cb2 + 4 * (lane >> 5), hbuf[(b + 1) & 1]);
            }
            if (cb < p.N) {
              float dg[16], dl[16], ps = 0.0f;
              glu_bwd_values_h<epi_act(EPI)>(hbuf[b & 1], rok, acc[i][j], p.clamp, p.alpha,
                                             p.gelu_tanh, sc, ps, dg, dl);
              if constexpr (RS)
                if (p.ds_part) ds_block_store(p.ds_part, p.ld_ds, cb >> 5, row, rok, ps);
              const int pg0 = (cb >> 5) * 64;
              mx_stage(Wt, lane, dg);
              mx_stage(Wt2, lane, dl);
              wave_lds_sync();
              mx_emit_two<typename EL::Fmt>(Wt, Wt2, lane, p, r0, r0, pg0, pg0 + 32, prow, prow,
                                            mlim, pe1);
              wave_lds_sync();
            }
          }
        });
      });
    } else if constexpr (epi_glu_bwd(EPI) && sizeof(SO) == 2) {
      // bf16 dGLU: the saved H of row block i + 1 (gate and linear values of
      // every column block) is requested before row block i is computed and
      // stored, so each block's load latency hides behind the previous block
      // instead of stalling every block in turn.
      u32x2 hr[2][TN][4][2];
      const SO* Hbase = reinterpret_cast<const SO*>(p.aux);
      auto hload = [&](int i, u32x2 (&buf)[TN][4][2]) {
        const int row = m0 + wm * C::WTM + 32 * i + (lane & 31);
        if (row < mlim) {
          const SO* Hrow = Hbase + (size_t)row * p.ld_aux;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = cw + 32 * j + 8 * g;
              const int pg = (col >> 5) * 64 + (col & 31);
              if (col < p.N) {
                buf[j][g][0] = *reinterpret_cast<const u32x2*>(Hrow + pg);
                buf[j][g][1] = *reinterpret_cast<const u32x2*>(Hrow + pg + 32);
              }
            }
        }
      };
      hload(0, hr[0]);
      if (kStagedDglu && !glu_direct) {
        if constexpr (kStagedDglu) {
        // dH through LDS: for each 32-row block the wave stages its 128 packed
        // dH columns (256-byte rows, chunk c of row r at c ^ (r & 15)) in the
        // ring slot that no wave reads any more, then writes whole rows, 16
        // bytes per lane.  Same values and rounding as the direct stores.
        // (Lane-dependent addresses are computed here, per tile, behind an
        // empty asm: hoisted out of the tile loop they would be spilled.)
        constexpr int CD = C::WTN * 2 * 2 / 16;   // 16-byte chunks per staged dH row
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int r = lane_e & 31, h = lane_e >> 5;
        u32x4* Ds = stage_ptr(nk) + wave * 32 * CD;
        char* Dr = reinterpret_cast<char*>(Ds) + r * CD * 16 + 8 * h;   // the lane's staged row
        const int wc0 = n0 + wn * C::WTN;     // the wave's first A column (a multiple of 64)
        SO* Dg = reinterpret_cast<SO*>(p.c);
        static_for<0, TM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const int rbase = m0 + wm * C::WTM + 32 * i;
          const int row = rbase + r;
          if (row < mlim) {
            const float sc = (RS && p.row_scale) ? p.row_scale[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int cb = wc0 + 32 * j;
              float ps = 0.0f;
              if (cb < p.N) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  float dg[4], dl[4];
                  glu_bwd_raw_group<epi_act(EPI)>(hr[i & 1][j][g], acc[i][j], g, p.clamp,
                                                  p.alpha, p.gelu_tanh, sc, ps, dg, dl);
                  // packed columns 64 j + 8 g + 4 h (gate) and 32 further (linear)
                  *reinterpret_cast<u32x2*>(Dr + ((8 * j + g) ^ (r & 15)) * 16) =
                      u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
                  *reinterpret_cast<u32x2*>(Dr + ((8 * j + 4 + g) ^ (r & 15)) * 16) =
                      u32x2{pack_bf16x2(dl[0], dl[1]), pack_bf16x2(dl[2], dl[3])};
                }
              }
              if constexpr (RS)
                if (p.ds_part) ds_block_store(p.ds_part, p.ld_ds, cb >> 5, row, cb < p.N, ps);
            }
          }
          // the next block's H is requested once this block's is used; its
          // latency hides behind the row stores below
          if constexpr (i + 1 < TM) hload(i + 1, hr[(i + 1) & 1]);
          wave_lds_sync();
#pragma unroll
          for (int it = 0; it < 32 * CD / 64; ++it) {
            const int rr = it * (64 / CD) + lane_e / CD, cc = lane_e % CD;
            const u32x4 v = Ds[rr * CD + (cc ^ (rr & 15))];
            const int orow = rbase + rr;
            if (orow < mlim && wc0 + 32 * (cc / 8) < p.N)
              *reinterpret_cast<u32x4*>(Dg + (size_t)orow * p.ldc + 2 * wc0 + cc * 8) = v;
          }
          wave_lds_sync();
        });
        }
      } else {
      static_for<0, TM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + 1 < TM) hload(i + 1, hr[(i + 1) & 1]);
        const int row = m0 + wm * C::WTM + 32 * i + (lane & 31);
        if (row < mlim) {
          SO* Drow = reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc;
          const float sc = (RS && p.row_scale) ? p.row_scale[row] : 1.0f;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            float ps = 0.0f;
            epi_glu_bwd_raw<epi_act(EPI)>(hr[i & 1][j], Drow, acc[i][j], cw + 32 * j, p.N,
                                          p.clamp, p.alpha, p.gelu_tanh, sc, ps);
            const int cb = n0 + wn * C::WTN + 32 * j;
            if constexpr (RS)
              if (p.ds_part) ds_block_store(p.ds_part, p.ld_ds, cb >> 5, row, cb < p.N, ps);
          }
        }
      });
      }
    } else if (kStagedGlu && !glu_direct) {
      if constexpr (kStagedGlu) {
      // FC1 + GLU through LDS: for each 32-row block the wave stages its 64
      // packed H columns (128-byte rows, chunk c of row r at c ^ ((r >> 1) &
      // 7)) and its 32 A columns (64-byte rows, chunk c at c ^ ((r >> 1) & 3))
      // in the ring slot that no wave reads any more (as the plain staged
      // epilogue below), then writes whole rows, 16 bytes per lane (H only
      // when it is saved).  Same values and rounding as epi_glu_fwd.
      constexpr int CH = C::WTN * 2 / 16;   // 16-byte chunks per staged H row
      constexpr int CA = C::WTN / 16;       // per staged A row
      u32x4* Hs = stage_ptr(nk) + wave * 32 * (CH + CA);
      u32x4* As = Hs + 32 * CH;
      char* Hb = reinterpret_cast<char*>(Hs);
      char* Ab = reinterpret_cast<char*>(As);
      auto hslot = [](int rr, int c) { return c ^ ((rr >> 1) & 7); };
      auto aslot = [](int rr, int c) { return c ^ ((rr >> 1) & 3); };
      const float* bias = p.bias ? p.bias + (size_t)e * p.ld_bias : nullptr;
      // lane-dependent addresses are computed here, per tile, behind an
      // empty asm: hoisted out of the tile loop they would be held (or
      // spilled) through the main loop
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      const int r = lane_e & 31, h = lane_e >> 5;
      const int wc0 = n0 + wn * C::WTN;     // the wave's first packed column (a multiple of 64)
      SO* Hg = reinterpret_cast<SO*>(p.aux);
      SO* Ag = reinterpret_cast<SO*>(p.c);
      static_for<0, TM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int rbase = m0 + wm * C::WTM + 32 * i;
        const int row_l = rbase + r;
        const float sc = (RS && p.row_scale && row_l < mlim) ? p.row_scale[row_l] : 1.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cl = 8 * g + 4 * h;       // gate column in the wave (linear: + 32)
          const int colg = wc0 + cl;
          const bool cok = colg < p.N;
          float gv[4], lv[4], o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc[i][0][4 * g + q] + ((bias && cok) ? bias[colg + q] : 0.0f);
            lv[q] = acc[i][1][4 * g + q] + ((bias && cok) ? bias[colg + 32 + q] : 0.0f);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float gt = gv[q], li = lv[q];
            if (p.clamp > 0.0f) {
              gt = fminf(gt, p.clamp);
              li = fminf(fmaxf(li, -p.clamp), p.clamp);
            }
            o[q] = act_value<epi_act(EPI)>(gt, p.alpha, p.gelu_tanh) * li * sc;
          }
          if (Hg) {
            *reinterpret_cast<u32x2*>(Hb + (r * CH + hslot(r, cl / 8)) * 16 + (cl % 8) * 2) =
                u32x2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
            *reinterpret_cast<u32x2*>(Hb + (r * CH + hslot(r, (cl + 32) / 8)) * 16 + (cl % 8) * 2) =
                u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
          }
          if (glu_a_direct) {
            if (row_l < mlim && cok) store4(Ag + (size_t)row_l * p.ldc + wc0 / 2 + cl, o);
          } else {
            *reinterpret_cast<u32x2*>(Ab + (r * CA + aslot(r, cl / 8)) * 16 + (cl % 8) * 2) =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          }
        }
        wave_lds_sync();
        if (Hg) {
#pragma unroll
          for (int it = 0; it < 32 * CH / 64; ++it) {
            const int rr = it * (64 / CH) + lane_e / CH, cc = lane_e % CH;
            const u32x4 v = Hs[rr * CH + hslot(rr, cc)];
            const int row = rbase + rr, col = wc0 + cc * 8;
            if (row < mlim && col < p.N)
              *reinterpret_cast<u32x4*>(Hg + (size_t)row * p.ld_aux + col) = v;
          }
        }
#pragma unroll
        for (int it = 0; it < 32 * CA / 64; ++it) {
          if (glu_a_direct) break;
          const int rr = it * (64 / CA) + lane_e / CA, cc = lane_e % CA;
          const u32x4 v = As[rr * CA + aslot(rr, cc)];
          const int row = rbase + rr, col = wc0 / 2 + cc * 8;
          if (row < mlim && col < p.N / 2)
            *reinterpret_cast<u32x4*>(Ag + (size_t)row * p.ldc + col) = v;
        }
        wave_lds_sync();
      });
      }
    } else if (kStaged && !(GROUP == RAGGED_K && p.accumulate)) {
      if constexpr (kStaged) {
        // Plain epilogue through LDS: each wave stages 32 rows x WTN columns of
        // its tile at a time in a ring slot that no wave reads any more
        // (nk % STAGES onwards, up to STAGES - 1 slots: their last readers
        // passed the barrier of the last step, and no load is in flight into
        // them; the next tile's loads start after the tile barrier), then
        // writes whole rows -- 16 bytes per lane, a
        // row's WTN columns contiguous -- instead of 16-byte pieces of 32 rows
        // per store.  Chunk c (16 bytes) of staged row r sits at c ^ ((r >> 1)
        // & 7) for 128-byte rows or c ^ (r & 15) for 256-byte rows, so the
        // accumulator writes (32 rows, one chunk each) and the row reads touch
        // each bank at most twice.  Same values and rounding as the direct path.
        constexpr int OB = (int)sizeof(OT);
        constexpr int CPRW = C::WTN * OB / 16;     // 16-byte chunks per staged row
        constexpr int EPC = 16 / OB;               // elements per chunk
        constexpr int RPI = 64 / CPRW;             // staged rows per wave instruction
        auto slot = [](int r, int c) { return CPRW == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15)); };
        constexpr int SW = C::template stage_waves<OT>();
        u32x4* Wt = stage_ptr(nk + wave / SW) + (wave % SW) * 32 * CPRW;
        char* Wb = reinterpret_cast<char*>(Wt);
        const float* bias = (GROUP == RAGGED_M && p.bias) ? p.bias + (size_t)e * p.ld_bias : nullptr;
        OT* Cg = reinterpret_cast<OT*>(p.c);
        if constexpr (GROUP == RAGGED_K) Cg += (size_t)e * p.c_expert_stride;
        // the lane's staging addresses are computed here, per tile: hoisted
        // out of the tile loop they would be held (or spilled) through the
        // main loop
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int r = lane_e & 31, h = lane_e >> 5;
        static_for<0, TM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          static_for<0, TN>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int cl = 32 * j + 8 * g + 4 * h;   // column within the wave tile
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = acc[i][j][4 * g + q];
                if (bias && cw + 32 * j + 8 * g + q < p.N) v[q] += bias[cw + 32 * j + 8 * g + q];
              }
              if constexpr (OB == 2) {
                const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(Wb + (r * CPRW + slot(r, cl / 8)) * 16 + (cl % 8) * 2) = w;
              } else {
                Wt[r * CPRW + slot(r, cl / 4)] = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                       __float_as_uint(v[2]), __float_as_uint(v[3])};
              }
            }
          });
          wave_lds_sync();
#pragma unroll
          for (int it = 0; it < 32 / RPI; ++it) {
            const int rr = it * RPI + lane_e / CPRW, cc = lane_e % CPRW;
            const u32x4 v = Wt[rr * CPRW + slot(rr, cc)];
            const int row = m0 + wm * C::WTM + 32 * i + rr;
            const int col = n0 + wn * C::WTN + cc * EPC;
            if (row < mlim && col < p.N)
              *reinterpret_cast<u32x4*>(Cg + (size_t)row * p.ldc + col) = v;
          }
          wave_lds_sync();
        });
      }
    } else
    static_for<0, TM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = m0 + wm * C::WTM + 32 * i + (lane & 31);
      if (row < mlim) {
        static_for<0, TN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const int c0 = cw + 32 * j;
          if constexpr (EPI == EPI_STORE && GROUP == RAGGED_M) {
            epi_store<SO>(reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc,
                         p.bias ? p.bias + (size_t)e * p.ld_bias : nullptr, acc[i][j], c0, p.N);
          } else if constexpr (EPI == EPI_STORE) {
            epi_store_f32(reinterpret_cast<float*>(p.c) + (size_t)e * p.c_expert_stride +
                              (size_t)row * p.ldc,
                          acc[i][j], c0, p.N, p.accumulate);
          } else if constexpr (epi_glu_fwd(EPI)) {
            if constexpr ((j & 1) == 0)
              epi_glu_fwd<epi_act(EPI), SO>(
                  p.aux ? reinterpret_cast<SO*>(p.aux) + (size_t)row * p.ld_aux : nullptr,
                  reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc,
                  p.bias ? p.bias + (size_t)e * p.ld_bias : nullptr, acc[i][j], acc[i][j + 1],
                  c0, p.N, p.clamp, p.alpha, p.gelu_tanh,
                  (RS && p.row_scale) ? p.row_scale[row] : 1.0f);
          } else if constexpr (epi_glu_bwd(EPI)) {
            float ps = 0.0f;
            epi_glu_bwd<epi_act(EPI), SO>(
                reinterpret_cast<const SO*>(p.aux) + (size_t)row * p.ld_aux,
                reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc, acc[i][j], c0, p.N, p.clamp,
                p.alpha, p.gelu_tanh, (RS && p.row_scale) ? p.row_scale[row] : 1.0f, ps);
            if constexpr (RS)
              if (p.ds_part) ds_block_store(p.ds_part, p.ld_ds, c0 >> 5, row, c0 < p.N, ps);
          } else if constexpr (EPI == EPI_SRELU_FWD) {
            epi_srelu_fwd<SO>(
                p.aux ? reinterpret_cast<SO*>(p.aux) + (size_t)row * p.ld_aux : nullptr,
                reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc,
                p.bias ? p.bias + (size_t)e * p.ld_bias : nullptr, acc[i][j], c0, p.N, p.clamp,
                (RS && p.row_scale) ? p.row_scale[row] : 1.0f);
          } else if constexpr (EPI == EPI_SRELU_BWD) {
            float ps = 0.0f;
            epi_srelu_bwd<SO>(reinterpret_cast<const SO*>(p.aux) + (size_t)row * p.ld_aux,
                             reinterpret_cast<SO*>(p.c) + (size_t)row * p.ldc, acc[i][j], c0,
                             p.N, p.clamp, (RS && p.row_scale) ? p.row_scale[row] : 1.0f, ps);
            if constexpr (RS)
              if (p.ds_part) ds_block_store(p.ds_part, p.ld_ds, c0 >> 5, row, c0 < p.N, ps);
          }
        });
      }
    });
  }
}

// ------------------------------------------------------------------ launching

template <class EL, bool AKM, bool BKM, int GROUP, int EPI, class TL, bool GATHER = false,
          bool RS = false>
moe_status_t launch_gemm(const GemmArgs& p, int max_cus, hipStream_t s) {
  typedef GemmCfg<EL, EPI, TL> C;
  auto kern = grouped_gemm_kernel<EL, AKM, BKM, GROUP, EPI, TL, GATHER, RS>;
  static int occ[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  if (occ[dev] == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)C::LDS_BYTES) != hipSuccess)
      return MOE_ERR_HIP;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, C::THREADS, C::LDS_BYTES) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    occ[dev] = n;
  }
  int cus = device_cu_count();
  if (max_cus > 0 && max_cus < cus) cus = max_cus;
  int grid = cus * occ[dev];
  grid = grid < 8 ? 8 : grid / 8 * 8;  // the XCD-grouped block order needs a multiple of 8
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, p);
  return launch_status();
}

// Tile policies.  Large bf16 problems take 256 x 256 tiles with a two-stage
// ring of 128-byte k-steps (64 KB each):
//  - plain epilogue, both operands K-contiguous (FC2): 16 waves in a 4 x 4
//    grid (64 x 64 per wave) with the pinned MFMA / LDS-read interleave;
//  - plain epilogue with an MN-contiguous B (dgrads, weight gradients): 8
//    waves in two ping-pong groups (128 x 64 per wave);
//  - gated epilogues: 8 waves in 2 x 4 with the pinned interleave (their
//    extra registers do not fit under the 16-wave limit of 128 VGPRs).
// Each choice is the fastest of a same-process sweep at the DeepSeek-V3-like
// shard.  Small or narrow problems take 128 x 128, fp32 takes 64 x 128.
// A library built with -DMOE_GEMM_TUNING (for tuning sweeps only) reads
// MOE_GEMM_TILE=<n> from the environment and takes variant n of the list
// below for bf16 instead; the product library never reads the environment.
typedef Tile<256, 256, 4, 4, 128, 2, 1> TBig;
typedef Tile<256, 256, 2, 4, 128, 2, 1> TBigGlu;
typedef Tile<256, 256, 2, 4, 128, 2, 2> TBigPingPong;
typedef Tile<128, 128, 2, 2, 128, 2> TSmall;
typedef Tile<64, 128, 2, 2, 128, 2> TF32;

inline int tile_variant() {
#ifdef MOE_GEMM_TUNING
  const char* v = getenv("MOE_GEMM_TILE");
  return v ? atoi(v) : -1;
#else
  return -1;
#endif
}

#ifdef MOE_GEMM_TUNING
// Weight-gradient ring shapes for tuning sweeps (MOE_GEMM_WGRAD=<n>).
inline int wgrad_variant() {
  const char* v = getenv("MOE_GEMM_WGRAD");
  return v ? atoi(v) : 0;
}
#endif

template <class EL, bool AKM, bool BKM, int GROUP, int EPI, bool GATHER = false,
          bool RS = false>
moe_status_t dispatch_tiles(const GemmArgs& p, bool big, int max_cus, hipStream_t s) {
  if constexpr (sizeof(typename EL::storage) == 4) {
    return launch_gemm<EL, AKM, BKM, GROUP, EPI, TF32, GATHER, RS>(p, max_cus, s);
  } else {
    constexpr bool kSweep =
        !GATHER && !RS && (EPI == EPI_STORE || EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD);
    if constexpr (kSweep) {
      switch (tile_variant()) {
        case 0: return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBig>(p, max_cus, s);
        case 1: return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBigGlu>(p, max_cus, s);
        case 2: return launch_gemm<EL, AKM, BKM, GROUP, EPI, Tile<256, 256, 4, 4, 128, 2, 0>>(p, max_cus, s);
        case 3: return launch_gemm<EL, AKM, BKM, GROUP, EPI, TSmall>(p, max_cus, s);
        case 4: return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBigPingPong>(p, max_cus, s);
        default: break;
      }
    }
#ifdef MOE_GEMM_TUNING
    if constexpr (GROUP == RAGGED_K && !AKM && !BKM && EPI == EPI_STORE && !RS) {
      if (big) switch (wgrad_variant()) {
          case 1:  // 48-k steps, three-deep ring (144 KB)
            return launch_gemm<EL, AKM, BKM, GROUP, EPI, Tile<256, 256, 2, 4, 96, 3, 2>, GATHER>(
                p, max_cus, s);
          case 2:  // 32-k steps, four-deep ring (128 KB)
            return launch_gemm<EL, AKM, BKM, GROUP, EPI, Tile<256, 256, 2, 4, 64, 4, 2>, GATHER>(
                p, max_cus, s);
          case 3:  // 16 waves (64 x 64 each) in two ping-pong groups, 32-k steps, 4-deep
            return launch_gemm<EL, AKM, BKM, GROUP, EPI, Tile<256, 256, 4, 4, 64, 4, 2>, GATHER>(
                p, max_cus, s);
          case 4:  // the same with a two-deep ring
            return launch_gemm<EL, AKM, BKM, GROUP, EPI, Tile<256, 256, 4, 4, 64, 2, 2>, GATHER>(
                p, max_cus, s);

          default:
            break;
        }
    }
#endif
    if (!big) return launch_gemm<EL, AKM, BKM, GROUP, EPI, TSmall, GATHER, RS>(p, max_cus, s);
    if constexpr (epi_glu_fwd(EPI) || epi_glu_bwd(EPI))
      return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBigGlu, GATHER, RS>(p, max_cus, s);
    else if constexpr (!BKM)
      return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBigPingPong, GATHER, RS>(p, max_cus, s);
    else return launch_gemm<EL, AKM, BKM, GROUP, EPI, TBig, GATHER, RS>(p, max_cus, s);
  }
}

// MXFP8 operands: 8 waves at 256 x 256 (one scale-word load per wave), or
// 4 waves at 128 x 128 for small problems.
typedef Tile<256, 256, 2, 4, 128, 2, 1> TMxBig;
typedef Tile<128, 128, 2, 2, 128, 2> TMxSmall;
// MXFP4: 64-byte steps (128 k, one scale word) in a three-deep ring.
typedef Tile<256, 256, 2, 4, 64, 3, 1> TMx4Big;
typedef Tile<128, 128, 2, 2, 64, 3> TMx4Small;

template <int GROUP, int EPI, bool RS = false>
moe_status_t dispatch_mx(const GemmArgs& p, bool big, int max_cus, hipStream_t s, int dtype) {
  if (dtype == MOE_E2M1) {
    if (big) return launch_gemm<MX4, true, true, GROUP, EPI, TMx4Big, false, RS>(p, max_cus, s);
    return launch_gemm<MX4, true, true, GROUP, EPI, TMx4Small, false, RS>(p, max_cus, s);
  }
  if (big) return launch_gemm<MX8, true, true, GROUP, EPI, TMxBig, false, RS>(p, max_cus, s);
  return launch_gemm<MX8, true, true, GROUP, EPI, TMxSmall, false, RS>(p, max_cus, s);
}

// The feature-scaling variant when row_scale or ds_part is set.
template <int GROUP, int EPI>
moe_status_t dispatch_mx_rs(const GemmArgs& p, bool big, int max_cus, hipStream_t s, int dtype) {
  if (p.row_scale || p.ds_part) return dispatch_mx<GROUP, EPI, true>(p, big, max_cus, s, dtype);
  return dispatch_mx<GROUP, EPI>(p, big, max_cus, s, dtype);
}

// p.gather selects the gather-fused loaders, built for FC1's forward (rows
// of A) and the weight gradient (k-rows of B) only.
template <bool AKM, bool BKM, int GROUP, int EPI, bool RS = false>
moe_status_t dispatch_rs(int dtype, const GemmArgs& p, bool big, int max_cus, hipStream_t s) {
  constexpr bool kGather =
      (GROUP == RAGGED_M && AKM && (epi_glu_fwd(EPI) || EPI == EPI_SRELU_FWD)) ||
      (GROUP == RAGGED_K && !BKM && EPI == EPI_STORE);
  if constexpr (kGather) {
    if (p.gather) {
      if (dtype == MOE_BF16)
        return dispatch_tiles<BF16, AKM, BKM, GROUP, EPI, true, RS>(p, big, max_cus, s);
      return dispatch_tiles<F32, AKM, BKM, GROUP, EPI, true, RS>(p, big, max_cus, s);
    }
  } else {
    if (p.gather) return MOE_ERR_UNSUPPORTED;
  }
  if (dtype == MOE_BF16)
    return dispatch_tiles<BF16, AKM, BKM, GROUP, EPI, false, RS>(p, big, max_cus, s);
  return dispatch_tiles<F32, AKM, BKM, GROUP, EPI, false, RS>(p, big, max_cus, s);
}

// Plain epilogues ignore the feature-scaling fields; the GLU / sReLU ones take
// their feature-scaling variant when row_scale or ds_part is set.
template <bool AKM, bool BKM, int GROUP, int EPI>
moe_status_t dispatch(int dtype, const GemmArgs& p, bool big, int max_cus, hipStream_t s) {
  if constexpr (EPI != EPI_STORE) {
    if (p.row_scale || p.ds_part)
      return dispatch_rs<AKM, BKM, GROUP, EPI, true>(dtype, p, big, max_cus, s);
  }
  return dispatch_rs<AKM, BKM, GROUP, EPI>(dtype, p, big, max_cus, s);
}

// Band heights 4 (6 for the weight gradients, whose FC2 launch measured 5 %
// faster with it at the DeepSeek-V3-size shard) and the weight gradients'
// alternating tile order.  (A -DMOE_GEMM_TUNING build lets MOE_GEMM_GM and
// MOE_GEMM_GM_K override the band heights,
// MOE_GEMM_SNAKE=0 turn the alternating order off and MOE_GEMM_GLU_DIRECT=1
// (2) store the FC1 + GLU outputs (A) without the LDS staging, for tuning
// sweeps.)
inline GemmArgs zero_args() {
  GemmArgs p;
  memset(&p, 0, sizeof(p));
  p.alpha = 1.0f;
  p.gm = 4;
  p.gm_k = 6;
  p.snake = 1;
#ifdef MOE_GEMM_TUNING
  if (const char* v = getenv("MOE_GEMM_GM")) {
    int g = atoi(v);
    if (g >= 1 && g <= 64) p.gm = g;
  }
  if (const char* v = getenv("MOE_GEMM_GM_K")) {
    int g = atoi(v);
    if (g >= 1 && g <= 64) p.gm_k = g;
  }
  if (const char* v = getenv("MOE_GEMM_SNAKE")) p.snake = atoi(v) != 0;
  if (const char* v = getenv("MOE_GEMM_GLU_DIRECT")) p.glu_direct = atoi(v);
#endif
  return p;
}

// A problem is "big" when the average expert has at least 256 rows and the
// output is wide enough to give every compute unit several 256-wide tiles.
inline bool big_ragged_m(int R, int E, int N) { return R >= 256 * E && N >= 1024; }
inline bool big_ragged_k(int R, int E, int M, int N) {
  return R >= 256 * E && (long long)M * N >= 1024LL * 1024;
}

}  // namespace moe

using namespace moe;

// An MXFP8 GEMM operand with reduction length K: ld a multiple of 128 (whole
// scale words per k-step) and at least K.
// An MX output field of an argument struct, or NULL when the caller's struct
// predates it.
template <class A>
inline moe_mx_t* mx_out_field(const A* a, moe_mx_t* const A::*f) {
  const size_t end = (size_t)(reinterpret_cast<const char*>(&(a->*f)) -
                              reinterpret_cast<const char*>(a)) + sizeof(moe_mx_t*);
  return a->struct_size >= end ? a->*f : nullptr;
}

// The gather index of an argument struct, or NULL when the caller's struct
// predates the field.
template <class A>
inline const int32_t* gather_field(const A* a, const int32_t* const A::*f) {
  const size_t end = (size_t)(reinterpret_cast<const char*>(&(a->*f)) -
                              reinterpret_cast<const char*>(a)) + sizeof(const int32_t*) +
                     sizeof(int);
  return a->struct_size >= end ? a->*f : nullptr;
}
// An optional pointer field of an argument struct, or NULL when the caller's
// struct predates it.
template <class A>
inline const void* ptr_field(const A* a, const void* const A::*f) {
  const size_t end = (size_t)(reinterpret_cast<const char*>(&(a->*f)) -
                              reinterpret_cast<const char*>(a)) + sizeof(const void*);
  return a->struct_size >= end ? a->*f : nullptr;
}
// A field appended to an argument struct: its value when struct_size covers
// it, else zero (callers built against an older header).
template <class A, class T>
inline T opt_field(const A* a, T A::*f) {
  const size_t end = (size_t)(reinterpret_cast<const char*>(&(a->*f)) -
                              reinterpret_cast<const char*>(a)) + sizeof(T);
  return a->struct_size >= end ? a->*f : T{};
}

// Feature-scaling gradient: ds[r] = sum over the 32-column blocks b, in
// order, of part[b * R + r] for rows below offsets[E]; zero past it.
__global__ void __launch_bounds__(256) ds_reduce_kernel(const float* __restrict__ part, int nb,
                                                        const int32_t* __restrict__ offsets,
                                                        int E, int R, float* __restrict__ ds) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  float v = 0.0f;
  if (r < offsets[E])
    for (int b = 0; b < nb; ++b) v += part[(size_t)b * R + r];
  ds[r] = v;
}

// Sets the feature-scaling fields of p from a glu_bwd argument struct;
// returns the d_row_scale output (nullable) or an argument error.
inline moe_status_t set_row_scale_bwd(GemmArgs& p, const moe_glu_bwd_args_t* a, float** ds) {
  p.row_scale = opt_field(a, &moe_glu_bwd_args_t::row_scale);
  *ds = opt_field(a, &moe_glu_bwd_args_t::d_row_scale);
  if (*ds) {
    void* ws = opt_field(a, &moe_glu_bwd_args_t::ws);
    if (!ws || opt_field(a, &moe_glu_bwd_args_t::ws_bytes) <
                   moe_glu_bwd_workspace_size(a->R, a->f))
      return MOE_ERR_WORKSPACE;
    p.ds_part = static_cast<float*>(ws);
    p.ld_ds = a->R;
  }
  return MOE_OK;
}

// After the dGLU GEMM on the same stream: the rows' sums of the partials.
inline moe_status_t ds_reduce(const GemmArgs& p, int f, float* ds, hipStream_t s) {
  if (!ds) return MOE_OK;
  hipLaunchKernelGGL(ds_reduce_kernel, dim3((p.R + 255) / 256), dim3(256), 0, s, p.ds_part,
                     f / 32, p.offsets, p.E, p.R, ds);
  return launch_status();
}
// A gathered source [rows, cols] must be addressable by 31-bit byte offsets.
inline bool gather_fits(long long rows, long long cols, int dtype) {
  return rows > 0 && rows * cols * (long long)dtype_size(dtype) <= 0x7ffffff0LL;
}

inline bool mx_in_ok(const moe_mx_t* m, long long K) {
  return m && m->data && m->scale && m->ld >= K && m->ld % 128 == 0 && aligned16(m->data) &&
         aligned16(m->scale);
}
inline bool mx_out_ok(const moe_mx_t* m, long long n) {
  return m && m->data && m->scale && m->ld >= n && m->ld % 32 == 0 && aligned16(m->data);
}
// Bytes per code row: E4M3 one per element, E2M1 two elements per byte.
inline long long mx_row_bytes(const moe_mx_t* m, int dtype) {
  return dtype == MOE_E2M1 ? m->ld / 2 : m->ld;
}
inline int mx_epb(int dtype) { return dtype == MOE_E2M1 ? 2 : 1; }

inline void set_mx_a(GemmArgs& p, const moe_mx_t* m, int dtype) {
  p.a = m->data;
  p.lda = mx_row_bytes(m, dtype);
  p.sa = m->scale;
  p.slda = m->ld / 32;
}
inline void set_mx_b(GemmArgs& p, const moe_mx_t* m, long long rows_per_expert, int dtype) {
  p.b = m->data;
  p.ldb = mx_row_bytes(m, dtype);
  p.sb = m->scale;
  p.sldb = m->ld / 32;
  p.b_expert_stride = rows_per_expert * p.ldb;
  p.sb_expert_stride = rows_per_expert * (m->ld / 32);
}
inline void set_mx_out(GemmArgs& p, moe_mx_t* row, moe_mx_t* col, const int32_t* pad) {
  if (row) {
    p.mxr = row->data;
    p.mxr_s = row->scale;
    p.ld_mxr = row->ld;
  }
  if (col) {
    p.mxc = col->data;
    p.mxc_s = col->scale;
    p.ld_mxc = col->ld;
  }
  p.pad_offsets = pad;
}

// MXFP8 FC1 + GLU (dtype == MOE_E4M3).
moe_status_t glu_fwd_mx(const moe_glu_fwd_args_t* a, hipStream_t s) {
  const int dt = a->dtype;
  MOE_CHECK_ARG(a->struct_size >= offsetof(moe_glu_fwd_args_t, src_row));
  MOE_CHECK_ARG(!gather_field(a, &moe_glu_fwd_args_t::src_row));
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU);
  MOE_CHECK_ARG(a->b1p == nullptr && a->d % 128 == 0);
  if (a->R == 0) return MOE_OK;
  const int n1 = 2 * a->f;
  MOE_CHECK_ARG(a->offsets && mx_in_ok(a->xp_mx, a->d) && mx_in_ok(a->w1_mx, a->d));
  MOE_CHECK_ARG(!a->a_row || mx_out_ok(a->a_row, a->f));
  MOE_CHECK_ARG(!a->a_col || (mx_out_ok(a->a_col, moe_mx_col_len(a->R, a->E)) && a->pad_offsets));
  MOE_CHECK_ARG(aligned16(a->h_out));
  GemmArgs p = zero_args();
  set_mx_a(p, a->xp_mx, dt);
  set_mx_b(p, a->w1_mx, n1, dt);
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = n1;
  p.K = a->d / mx_epb(dt);
  p.aux = a->h_out;
  p.ld_aux = n1;
  set_mx_out(p, a->a_row, a->a_col, a->pad_offsets);
  p.clamp = a->clamp;
  p.alpha = a->alpha;
  p.act = a->act;
  p.gelu_tanh = a->gelu_tanh;
  p.row_scale = opt_field(a, &moe_glu_fwd_args_t::row_scale);
  const bool big = big_ragged_m(a->R, a->E, n1);
  if (a->act == MOE_ACT_SWIGLU)
    return dispatch_mx_rs<RAGGED_M, EPI_SWIGLU_FWD>(p, big, a->max_cus, s, dt);
  return dispatch_mx_rs<RAGGED_M, EPI_GEGLU_FWD>(p, big, a->max_cus, s, dt);
}

moe_status_t gemm_fwd_mx(const moe_gemm_fwd_args_t* a, hipStream_t s) {
  const int dt = a->dtype;
  MOE_CHECK_ARG(a->struct_size >= offsetof(moe_gemm_fwd_args_t, y_mx));
  MOE_CHECK_ARG(a->b == nullptr && a->K % 128 == 0);
  if (a->R == 0) return MOE_OK;
  moe_mx_t* ymx = mx_out_field(a, &moe_gemm_fwd_args_t::y_mx);
  MOE_CHECK_ARG(a->offsets && (ymx ? mx_out_ok(ymx, a->N) && a->N % 32 == 0
                                   : (a->y && aligned16(a->y))));
  MOE_CHECK_ARG(mx_in_ok(a->a_mx, a->K) && mx_in_ok(a->w_mx, a->K));
  GemmArgs p = zero_args();
  set_mx_a(p, a->a_mx, dt);
  set_mx_b(p, a->w_mx, a->N, dt);
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = a->N;
  p.K = a->K / mx_epb(dt);
  p.c = a->y;
  p.ldc = a->N;
  set_mx_out(p, ymx, nullptr, nullptr);
  return dispatch_mx<RAGGED_M, EPI_STORE>(p, big_ragged_m(a->R, a->E, a->N), a->max_cus, s, dt);
}

moe_status_t glu_bwd_mx(const moe_glu_bwd_args_t* a, hipStream_t s) {
  const int dt = a->dtype;
  MOE_CHECK_ARG(a->struct_size >= offsetof(moe_glu_bwd_args_t, w2t));
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU);
  MOE_CHECK_ARG(a->d % 128 == 0);
  if (a->R == 0) return MOE_OK;
  const int n1 = 2 * a->f;
  MOE_CHECK_ARG(a->offsets && a->h && aligned16(a->h));
  MOE_CHECK_ARG(mx_in_ok(a->dy_mx, a->d) && mx_in_ok(a->w2t_mx, a->d));
  MOE_CHECK_ARG(!a->dh_row || mx_out_ok(a->dh_row, n1));
  MOE_CHECK_ARG(!a->dh_col ||
                (mx_out_ok(a->dh_col, moe_mx_col_len(a->R, a->E)) && a->pad_offsets));
  GemmArgs p = zero_args();
  set_mx_a(p, a->dy_mx, dt);
  set_mx_b(p, a->w2t_mx, a->f, dt);
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = a->f;
  p.K = a->d / mx_epb(dt);
  p.aux = const_cast<void*>(a->h);
  p.ld_aux = n1;
  set_mx_out(p, a->dh_row, a->dh_col, a->pad_offsets);
  p.clamp = a->clamp;
  p.alpha = a->alpha;
  p.act = a->act;
  p.gelu_tanh = a->gelu_tanh;
  float* ds = nullptr;
  if (const moe_status_t st = set_row_scale_bwd(p, a, &ds); st != MOE_OK) return st;
  const bool big = big_ragged_m(a->R, a->E, a->f);
  const moe_status_t st = a->act == MOE_ACT_SWIGLU
                              ? dispatch_mx_rs<RAGGED_M, EPI_SWIGLU_BWD>(p, big, a->max_cus, s, dt)
                              : dispatch_mx_rs<RAGGED_M, EPI_GEGLU_BWD>(p, big, a->max_cus, s, dt);
  return st != MOE_OK ? st : ds_reduce(p, a->f, ds, s);
}

moe_status_t gemm_bwd_mx(const moe_gemm_bwd_args_t* a, hipStream_t s) {
  const int dt = a->dtype;
  MOE_CHECK_ARG(a->struct_size >= offsetof(moe_gemm_bwd_args_t, a_src_row));
  MOE_CHECK_ARG(!gather_field(a, &moe_gemm_bwd_args_t::a_src_row));
  GemmArgs p = zero_args();
  p.E = a->E;
  if (a->mode == MOE_BWD_DGRAD) {
    // da [R, K] = g [R, N] @ w[e] [N, K] with w given transposed, [K, N] per expert
    MOE_CHECK_ARG(a->N % 128 == 0);
    if (a->R == 0) return MOE_OK;
    MOE_CHECK_ARG(a->offsets && mx_in_ok(a->g_mx, a->N) && mx_in_ok(a->w_mx, a->N));
    moe_mx_t* omx = mx_out_field(a, &moe_gemm_bwd_args_t::out_mx);
    MOE_CHECK_ARG(omx ? mx_out_ok(omx, a->K) && a->K % 32 == 0 : (a->out && aligned16(a->out)));
    set_mx_out(p, omx, nullptr, nullptr);
    set_mx_a(p, a->g_mx, dt);
    set_mx_b(p, a->w_mx, a->K, dt);
    p.offsets = a->offsets;
    p.R = a->R;
    p.N = a->K;
    p.K = a->N / mx_epb(dt);
    p.c = a->out;
    p.ldc = a->K;
    return dispatch_mx<RAGGED_M, EPI_STORE>(p, big_ragged_m(a->R, a->E, a->K), a->max_cus, s,
                                            dt);
  }
  // dw[e] [N, K] = g_col[:, seg e] @ a_col[:, seg e]^T; the k ranges are the
  // padded segments, so the offsets table is pad_offsets and R its bound
  MOE_CHECK_ARG(a->db == nullptr && a->pad_offsets && a->out && aligned16(a->out));
  MOE_CHECK_ARG(!mx_out_field(a, &moe_gemm_bwd_args_t::out_mx));
  const long long L = moe_mx_col_len(a->R, a->E);
  MOE_CHECK_ARG(mx_in_ok(a->g_mx, L) && mx_in_ok(a->a_mx, L));
  MOE_CHECK_ARG(L <= 0x7fffffff);
  set_mx_a(p, a->g_mx, dt);
  set_mx_b(p, a->a_mx, 0, dt);
  p.offsets = a->pad_offsets;
  p.R = (int)L;
  p.M = a->N;
  p.N = a->K;
  p.c = a->out;
  p.ldc = a->K;
  p.c_expert_stride = (long long)a->N * a->K;
  p.accumulate = a->accumulate;
  return dispatch_mx<RAGGED_K, EPI_STORE>(p, big_ragged_k(a->R, a->E, a->N, a->K), a->max_cus,
                                          s, dt);
}

extern "C" {

moe_status_t moe_grouped_gemm_glu_fwd(const moe_glu_fwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= offsetof(moe_glu_fwd_args_t, xp_mx));
  MOE_CHECK_ARG(a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1 || valid_dtype(a->dtype));
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->d > 0 && a->f > 0 && a->d % 32 == 0 && a->f % 32 == 0);
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU || a->act == MOE_ACT_SRELU);
  if (a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1)
    return glu_fwd_mx(a, reinterpret_cast<hipStream_t>(stream));
  if (a->R == 0) return MOE_OK;
  MOE_CHECK_ARG(a->xp && a->w1p && a->offsets && a->a_out);
  MOE_CHECK_ARG(aligned16(a->xp) && aligned16(a->w1p) && aligned16(a->a_out) &&
                aligned16(a->h_out) && aligned16(a->b1p));
  const bool gated = a->act != MOE_ACT_SRELU;
  const int n1 = gated ? 2 * a->f : a->f;
  GemmArgs p = zero_args();
  p.a = a->xp;
  p.b = a->w1p;
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = n1;
  p.K = a->d;
  p.lda = a->d;
  p.ldb = a->d;
  p.b_expert_stride = (long long)n1 * a->d;
  p.c = a->a_out;
  p.ldc = a->f;
  p.bias = a->b1p;
  p.ld_bias = n1;
  p.aux = a->h_out;
  p.ld_aux = n1;
  p.clamp = a->clamp;
  p.alpha = a->alpha;
  p.act = a->act;
  p.gelu_tanh = a->gelu_tanh;
  if (const int32_t* g = gather_field(a, &moe_glu_fwd_args_t::src_row)) {
    MOE_CHECK_ARG(gather_fits(a->src_rows, a->d, a->dtype));
    p.gather = g;
    p.gather_rows = a->src_rows;
  }
  p.row_scale = opt_field(a, &moe_glu_fwd_args_t::row_scale);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool big = big_ragged_m(a->R, a->E, n1);
  if (a->act == MOE_ACT_SWIGLU)
    return dispatch<true, true, RAGGED_M, EPI_SWIGLU_FWD>(a->dtype, p, big, a->max_cus, s);
  if (a->act == MOE_ACT_GEGLU)
    return dispatch<true, true, RAGGED_M, EPI_GEGLU_FWD>(a->dtype, p, big, a->max_cus, s);
  return dispatch<true, true, RAGGED_M, EPI_SRELU_FWD>(a->dtype, p, big, a->max_cus, s);
}

moe_status_t moe_grouped_gemm_fwd(const moe_gemm_fwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= offsetof(moe_gemm_fwd_args_t, a_mx));
  MOE_CHECK_ARG(a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1 || valid_dtype(a->dtype));
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->N > 0 && a->K > 0 && a->N % 8 == 0 && a->K % 8 == 0);
  if (a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1)
    return gemm_fwd_mx(a, reinterpret_cast<hipStream_t>(stream));
  MOE_CHECK_ARG(!mx_out_field(a, &moe_gemm_fwd_args_t::y_mx));
  if (a->R == 0) return MOE_OK;
  MOE_CHECK_ARG(a->a && a->w && a->offsets && a->y);
  MOE_CHECK_ARG(aligned16(a->a) && aligned16(a->w) && aligned16(a->y) && aligned16(a->b));
  GemmArgs p = zero_args();
  p.a = a->a;
  p.b = a->w;
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = a->N;
  p.K = a->K;
  p.lda = a->K;
  p.ldb = a->K;
  p.b_expert_stride = (long long)a->N * a->K;
  p.c = a->y;
  p.ldc = a->N;
  p.bias = a->b;
  p.ld_bias = a->N;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dispatch<true, true, RAGGED_M, EPI_STORE>(a->dtype, p, big_ragged_m(a->R, a->E, a->N),
                                                   a->max_cus, s);
}

moe_status_t moe_grouped_gemm_glu_bwd(const moe_glu_bwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= offsetof(moe_glu_bwd_args_t, dy_mx));
  MOE_CHECK_ARG(a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1 || valid_dtype(a->dtype));
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->d > 0 && a->f > 0 && a->d % 32 == 0 && a->f % 32 == 0);
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU || a->act == MOE_ACT_SRELU);
  if (a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1)
    return glu_bwd_mx(a, reinterpret_cast<hipStream_t>(stream));
  if (a->R == 0) return MOE_OK;
  const void* w2t = ptr_field(a, &moe_glu_bwd_args_t::w2t);
  MOE_CHECK_ARG(a->dy && (a->w2 || w2t) && a->h && a->offsets && a->dh);
  MOE_CHECK_ARG(aligned16(a->dy) && aligned16(w2t ? w2t : a->w2) && aligned16(a->h) &&
                aligned16(a->dh));
  const bool gated = a->act != MOE_ACT_SRELU;
  const int n1 = gated ? 2 * a->f : a->f;
  GemmArgs p = zero_args();
  p.a = a->dy;        // [R, d]: K = d
  p.b = a->w2;        // [E][d][f]: K = d rows, N = f contiguous
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  p.N = a->f;
  p.K = a->d;
  p.lda = a->d;
  p.ldb = a->f;
  p.b_expert_stride = (long long)a->d * a->f;
  p.c = a->dh;
  p.ldc = n1;
  p.aux = const_cast<void*>(a->h);
  p.ld_aux = n1;
  p.clamp = a->clamp;
  p.alpha = a->alpha;
  p.act = a->act;
  p.gelu_tanh = a->gelu_tanh;
  float* ds = nullptr;
  if (const moe_status_t st = set_row_scale_bwd(p, a, &ds); st != MOE_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool big = big_ragged_m(a->R, a->E, a->f);
  moe_status_t st;
  if (w2t) {
    p.b = w2t;        // [E][f][d]: N = f rows, K = d contiguous
    p.ldb = a->d;
    if (a->act == MOE_ACT_SWIGLU)
      st = dispatch<true, true, RAGGED_M, EPI_SWIGLU_BWD>(a->dtype, p, big, a->max_cus, s);
    else if (a->act == MOE_ACT_GEGLU)
      st = dispatch<true, true, RAGGED_M, EPI_GEGLU_BWD>(a->dtype, p, big, a->max_cus, s);
    else
      st = dispatch<true, true, RAGGED_M, EPI_SRELU_BWD>(a->dtype, p, big, a->max_cus, s);
  } else if (a->act == MOE_ACT_SWIGLU) {
    st = dispatch<true, false, RAGGED_M, EPI_SWIGLU_BWD>(a->dtype, p, big, a->max_cus, s);
  } else if (a->act == MOE_ACT_GEGLU) {
    st = dispatch<true, false, RAGGED_M, EPI_GEGLU_BWD>(a->dtype, p, big, a->max_cus, s);
  } else {
    st = dispatch<true, false, RAGGED_M, EPI_SRELU_BWD>(a->dtype, p, big, a->max_cus, s);
  }
  return st != MOE_OK ? st : ds_reduce(p, a->f, ds, s);
}

size_t moe_glu_bwd_workspace_size(int R, int f) {
  return R > 0 && f > 0 ? (size_t)((f + 31) / 32) * (size_t)R * sizeof(float) : 0;
}

moe_status_t moe_grouped_gemm_bwd(const moe_gemm_bwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= offsetof(moe_gemm_bwd_args_t, g_mx));
  MOE_CHECK_ARG(a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1 || valid_dtype(a->dtype));
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->N > 0 && a->K > 0 && a->N % 8 == 0 && a->K % 8 == 0);
  MOE_CHECK_ARG(a->mode == MOE_BWD_DGRAD || a->mode == MOE_BWD_WGRAD);
  if (a->dtype == MOE_E4M3 || a->dtype == MOE_E2M1)
    return gemm_bwd_mx(a, reinterpret_cast<hipStream_t>(stream));
  MOE_CHECK_ARG(a->out && aligned16(a->out));
  MOE_CHECK_ARG(!mx_out_field(a, &moe_gemm_bwd_args_t::out_mx));
  MOE_CHECK_ARG(a->g && a->offsets && aligned16(a->g));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemmArgs p = zero_args();
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  if (a->mode == MOE_BWD_DGRAD) {
    MOE_CHECK_ARG(!gather_field(a, &moe_gemm_bwd_args_t::a_src_row));
    if (a->R == 0) return MOE_OK;
    const void* wt = ptr_field(a, &moe_gemm_bwd_args_t::wt);
    MOE_CHECK_ARG((a->w || wt) && aligned16(wt ? wt : a->w));
    // da [R, K] = g [R, N] @ w[e] [N, K]:  GEMM M = rows, N' = K, K' = N
    p.a = a->g;
    p.b = a->w;
    p.N = a->K;
    p.K = a->N;
    p.lda = a->N;
    p.ldb = a->K;
    p.b_expert_stride = (long long)a->N * a->K;
    p.c = a->out;
    p.ldc = a->K;
    if (wt) {
      p.b = wt;       // [E][K][N]: N' = K rows, K' = N contiguous
      p.ldb = a->N;
      return dispatch<true, true, RAGGED_M, EPI_STORE>(a->dtype, p,
                                                       big_ragged_m(a->R, a->E, a->K),
                                                       a->max_cus, s);
    }
    return dispatch<true, false, RAGGED_M, EPI_STORE>(a->dtype, p,
                                                      big_ragged_m(a->R, a->E, a->K),
                                                      a->max_cus, s);
  }
  MOE_CHECK_ARG(a->a && aligned16(a->a));
  // dw[e] [N, K] = g[seg]^T [N, rows] @ a[seg] [rows, K]:  GEMM M = N, N' = K, K' = rows
  p.a = a->g;
  p.b = a->a;
  p.M = a->N;
  p.N = a->K;
  p.lda = a->N;
  p.ldb = a->K;
  p.c = a->out;
  p.ldc = a->K;
  p.c_expert_stride = (long long)a->N * a->K;
  p.accumulate = a->accumulate;
  if (const int32_t* g = gather_field(a, &moe_gemm_bwd_args_t::a_src_row)) {
    MOE_CHECK_ARG(gather_fits(a->a_src_rows, a->K, a->dtype));
    p.gather = g;
    p.gather_rows = a->a_src_rows;
  }
  moe_status_t st = dispatch<false, false, RAGGED_K, EPI_STORE>(
      a->dtype, p, big_ragged_k(a->R, a->E, a->N, a->K), a->max_cus, s);
  if (st != MOE_OK || !a->db) return st;
  return launch_segment_colsum(a->dtype, a->g, a->offsets, a->E, a->R, a->N, a->db,
                               a->accumulate, s);
}

}  // extern "C"
