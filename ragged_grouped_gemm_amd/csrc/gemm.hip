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
//    LDS and walks the tiles tile = vb, vb + grid, ...  The virtual id vb
//    groups consecutive tiles on one XCD (blocks are dealt round-robin over
//    the 8 XCDs), and tiles are ordered in bands of GM M-tiles so the
//    workgroups of an XCD share A rows and B columns in its L2.
//  * Two grouping modes: RAGGED_M (FC1, FC2, dgrads: M = rows of an expert,
//    B = that expert's weight) and RAGGED_K (weight gradients: K = rows of an
//    expert; experts visited largest first so the long tiles start early).
//  * Tiles of BM x BN x (128 bytes of K), double-buffered in LDS.  Every LDS
//    row holds 128 bytes of K as eight 16-byte chunks, chunk c of row r stored
//    at slot c ^ (r & 7), so a quarter-wave reading eight rows at one chunk
//    hits all 32 banks.  K-contiguous operands are copied as 16-byte chunks;
//    MN-contiguous operands (the transposed operands of dgrad / wgrad) are
//    loaded as VEC x VEC element blocks and transposed in registers before the
//    LDS store, so the MFMA loop always reads K-contiguous fragments.
//  * MFMA v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32),
//    fp32 accumulation.  The MFMA is issued with B as the first operand, so a
//    lane's 16 accumulators hold 4 runs of 4 consecutive output columns of one
//    row: the epilogue writes 8- or 16-byte vectors, and the gate and linear
//    halves of a GLU pair sit in the same lane at the same positions.
#include "common.hpp"

#include <math.h>

namespace moe {

enum { EPI_STORE = 0, EPI_GLU_FWD = 1, EPI_GLU_BWD = 2, EPI_SRELU_FWD = 3, EPI_SRELU_BWD = 4 };
enum { RAGGED_M = 0, RAGGED_K = 1 };

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
};

// ------------------------------------------------------------------ activations

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ float act_fwd(float g, int act, float alpha, int gtanh) {
  if (act == MOE_ACT_SWIGLU) return g * sigm(alpha * g);
  if (act == MOE_ACT_GEGLU) {
    if (gtanh) {
      const float c = 0.7978845608028654f;
      return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
    }
    return 0.5f * g * (1.0f + erff(g * 0.7071067811865476f));
  }
  float r = fmaxf(g, 0.0f);  // squared ReLU
  return r * r;
}

__device__ __forceinline__ float act_bwd(float g, int act, float alpha, int gtanh) {
  if (act == MOE_ACT_SWIGLU) {
    float s = sigm(alpha * g);
    return s + alpha * g * s * (1.0f - s);
  }
  if (act == MOE_ACT_GEGLU) {
    if (gtanh) {
      const float c = 0.7978845608028654f;
      float th = tanhf(c * (g + 0.044715f * g * g * g));
      return 0.5f * (1.0f + th) + 0.5f * g * (1.0f - th * th) * c * (1.0f + 0.134145f * g * g);
    }
    return 0.5f * (1.0f + erff(g * 0.7071067811865476f)) +
           g * expf(-0.5f * g * g) * 0.3989422804014327f;
  }
  return 2.0f * fmaxf(g, 0.0f);
}

// ------------------------------------------------------------------ tile loaders

// K-contiguous operand: ROWS x 128 bytes of K from X[row][k] (row stride ld).
template <class EL, int ROWS, int THREADS>
struct LoaderK {
  typedef typename EL::storage S;
  static constexpr int NCH = ROWS * 8;
  static constexpr int PER = (NCH + THREADS - 1) / THREADS;
  u32x4 r[PER];

  __device__ __forceinline__ void load(const S* X, long long ld, int r0, int rlim, int k0,
                                       int klim, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * THREADS;
      int row = q >> 3, c = q & 7;
      int gr = r0 + row, gk = k0 + c * EL::VEC;
      u32x4 v = {0u, 0u, 0u, 0u};
      if ((NCH % THREADS == 0 || q < NCH) && gr < rlim && gk < klim)
        v = *reinterpret_cast<const u32x4*>(X + (size_t)gr * ld + gk);
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * THREADS;
      if (NCH % THREADS == 0 || q < NCH) {
        int row = q >> 3, c = q & 7;
        lds[row * 8 + (c ^ (row & 7))] = r[i];
      }
    }
  }
};

// MN-contiguous operand: X[k][mn] (row stride ld); the tile covers ROWS values
// of mn and 128 bytes of k.  A job is a VEC(k) x VEC(mn) block: VEC 16-byte
// loads along mn, transposed in registers into VEC 16-byte chunks along k.
template <class EL, int ROWS, int THREADS>
struct LoaderMN {
  typedef typename EL::storage S;
  static constexpr int V = EL::VEC;
  static constexpr int JOBS = (ROWS / V) * 8;
  static constexpr int PER = (JOBS + THREADS - 1) / THREADS;
  u32x4 r[PER][V];

  __device__ __forceinline__ void load(const S* X, long long ld, int c0, int clim, int k0,
                                       int klim, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int job = tid + i * THREADS;
      int kb = job & 7, mb = job >> 3;
      int gmn = c0 + mb * V;
      bool ok = (JOBS % THREADS == 0 || job < JOBS) && gmn < clim;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        int gk = k0 + kb * V + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok && gk < klim) v = *reinterpret_cast<const u32x4*>(X + (size_t)gk * ld + gmn);
        r[i][j] = v;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int job = tid + i * THREADS;
      if (JOBS % THREADS == 0 || job < JOBS) {
        int kb = job & 7, mb = job >> 3;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          u32x4 o;
          if constexpr (V == 8) {
            // element e of each of the 8 k-rows: bf16 halves of dword e/2
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              uint32_t lo = r[i][2 * h][e >> 1], hi = r[i][2 * h + 1][e >> 1];
              o[h] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
          } else {
#pragma unroll
            for (int h = 0; h < 4; ++h) o[h] = r[i][h][e];
          }
          int row = mb * V + e;
          lds[row * 8 + (kb ^ (row & 7))] = o;
        }
      }
    }
  }
};

template <bool KMAJOR, class EL, int ROWS, int THREADS>
struct Loader;
template <class EL, int ROWS, int THREADS>
struct Loader<true, EL, ROWS, THREADS> : LoaderK<EL, ROWS, THREADS> {};
template <class EL, int ROWS, int THREADS>
struct Loader<false, EL, ROWS, THREADS> : LoaderMN<EL, ROWS, THREADS> {};

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

// ------------------------------------------------------------------ the kernel

template <class EL, bool AKM, bool BKM, int GROUP, int EPI, int BM, int BN, int WGM, int WGN>
struct GemmCfg {
  static constexpr int THREADS = WGM * WGN * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int BK = 128 / sizeof(typename EL::storage);
  static constexpr int GM = 8;  // M-tiles per band of the tile order
  static constexpr size_t LDS_BYTES = 2 * (size_t)(BM + BN) * 128;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(EPI != EPI_GLU_FWD || WTN % 64 == 0, "GLU pairs need 64-column wave tiles");
};

template <class EL, bool AKM, bool BKM, int GROUP, int EPI, int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(WGM * WGN * 64)
    grouped_gemm_kernel(GemmArgs p) {
  typedef GemmCfg<EL, AKM, BKM, GROUP, EPI, BM, BN, WGM, WGN> C;
  typedef typename EL::storage S;
  constexpr int THREADS = C::THREADS, TM = C::TM, TN = C::TN, BK = C::BK;
  extern __shared__ u32x4 smem[];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_tab[MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int E = p.E;

  // ---- tile table (device-side shapes) ----
  for (int e = tid; e <= E; e += THREADS) {
    int o = p.offsets[e];
    s_off[e] = o < 0 ? 0 : (o > p.R ? p.R : o);
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
  u32x4* buf0 = smem;
  u32x4* buf1 = smem + (BM + BN) * 8;

  for (int tile = vb; tile < total; tile += G) {
    // ---- decode the tile ----
    int e, m0, n0, mlim, kbeg, kend;
    if constexpr (GROUP == RAGGED_M) {
      const int total_m = s_tab[E];
      const int span = C::GM * nN;
      int band = tile / span, in = tile - band * span;
      int first = band * C::GM;
      int gsz = min(total_m - first, C::GM);
      int gm = first + in % gsz;
      int nt = in / gsz;
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (s_tab[mid] <= gm) lo = mid; else hi = mid;
      }
      e = lo;
      m0 = s_off[e] + (gm - s_tab[e]) * BM;
      mlim = s_off[e + 1];
      n0 = nt * BN;
      kbeg = 0;
      kend = p.K;
    } else {
      const int per = mt_k * nt_k;
      int slot = tile / per, in = tile - slot * per;
      e = s_tab[slot];
      const int span = C::GM * nt_k;
      int band = in / span, r = in - band * span;
      int first = band * C::GM;
      int gsz = min(mt_k - first, C::GM);
      m0 = (first + r % gsz) * BM;
      n0 = (r / gsz) * BN;
      mlim = p.M;
      kbeg = s_off[e];
      kend = max(s_off[e + 1], kbeg);
    }

    // ---- main loop ----
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const S* A = reinterpret_cast<const S*>(p.a);
    const S* B = reinterpret_cast<const S*>(p.b);
    if constexpr (GROUP == RAGGED_M) B += (size_t)e * p.b_expert_stride;
    Loader<AKM, EL, BM, THREADS> la;
    Loader<BKM, EL, BN, THREADS> lb;
    const int nk = (kend - kbeg + BK - 1) / BK;

    auto load_tiles = [&](int k0) {
      if constexpr (GROUP == RAGGED_M) {
        la.load(A, p.lda, m0, mlim, k0, kend, tid);     // A [R][K]
      } else {
        la.load(A, p.lda, m0, mlim, k0, kend, tid);     // A [rows=K][M]
      }
      lb.load(B, p.ldb, n0, p.N, k0, kend, tid);
    };

    if (nk > 0) {
      load_tiles(kbeg);
      __syncthreads();  // the previous tile's readers are done with buf0
      la.store(buf0, tid);
      lb.store(buf0 + BM * 8, tid);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        u32x4* cur = (kt & 1) ? buf1 : buf0;
        u32x4* nxt = (kt & 1) ? buf0 : buf1;
        if (kt + 1 < nk) load_tiles(kbeg + (kt + 1) * BK);
        const u32x4* As = cur;
        const u32x4* Bs = cur + BM * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch = 2 * s + (lane >> 5);
          u32x4 af[TM], bfr[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            int row = wm * C::WTM + 32 * i + (lane & 31);
            af[i] = As[row * 8 + (ch ^ (row & 7))];
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            int row = wn * C::WTN + 32 * j + (lane & 31);
            bfr[j] = Bs[row * 8 + (ch ^ (row & 7))];
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) mma(acc[i][j], bfr[j], af[i], EL());
        }
        if (kt + 1 < nk) {
          la.store(nxt, tid);
          lb.store(nxt + BM * 8, tid);
        }
        __syncthreads();
      }
    }

    // ---- epilogue: lane holds rows (lane & 31) + 32 i, columns 32 j + 8 g + 4 h + q ----
    const int h4 = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = m0 + wm * C::WTM + 32 * i + (lane & 31);
      if (row >= mlim) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * C::WTN + 32 * j + 8 * g + h4;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
          if constexpr (EPI == EPI_STORE && GROUP == RAGGED_M) {
            if (col < p.N) {
              if (p.bias) {
                const float* bb = p.bias + (size_t)e * p.ld_bias + col;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] += bb[q];
              }
              store4(reinterpret_cast<S*>(p.c) + (size_t)row * p.ldc + col, v);
            }
          } else if constexpr (EPI == EPI_STORE && GROUP == RAGGED_K) {
            if (col < p.N) {
              float* cp = reinterpret_cast<float*>(p.c) + (size_t)e * p.c_expert_stride +
                          (size_t)row * p.ldc + col;
              if (p.accumulate) {
                float o[4];
                load4(cp, o);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] += o[q];
              }
              store4(cp, v);
            }
          } else if constexpr (EPI == EPI_GLU_FWD) {
            // j even: gate chunk; j + 1: the matching linear chunk (32 columns later)
            if ((j & 1) == 0 && col < p.N) {
              float lv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) lv[q] = acc[i][j + 1][4 * g + q];
              const int colL = col + 32;
              if (p.bias) {
                const float* bb = p.bias + (size_t)e * p.ld_bias;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  v[q] += bb[col + q];
                  lv[q] += bb[colL + q];
                }
              }
              if (p.aux) {
                S* H = reinterpret_cast<S*>(p.aux) + (size_t)row * p.ld_aux;
                store4(H + col, v);
                store4(H + colL, lv);
              }
              float o[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float gt = v[q], li = lv[q];
                if (p.clamp > 0.0f) {
                  gt = fminf(gt, p.clamp);
                  li = fminf(fmaxf(li, -p.clamp), p.clamp);
                }
                o[q] = act_fwd(gt, p.act, p.alpha, p.gelu_tanh) * li;
              }
              const int acol = (col >> 6) * 32 + (col & 31);
              store4(reinterpret_cast<S*>(p.c) + (size_t)row * p.ldc + acol, o);
            }
          } else if constexpr (EPI == EPI_GLU_BWD) {
            if (col < p.N) {
              const int pg = (col >> 5) * 64 + (col & 31), pl = pg + 32;
              const S* H = reinterpret_cast<const S*>(p.aux) + (size_t)row * p.ld_aux;
              float hg[4], hl[4], dg[4], dl[4];
              load4(H + pg, hg);
              load4(H + pl, hl);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float gt = hg[q], li = hl[q], mg = 1.0f, ml = 1.0f;
                if (p.clamp > 0.0f) {
                  mg = gt <= p.clamp ? 1.0f : 0.0f;
                  ml = (li >= -p.clamp && li <= p.clamp) ? 1.0f : 0.0f;
                  gt = fminf(gt, p.clamp);
                  li = fminf(fmaxf(li, -p.clamp), p.clamp);
                }
                dg[q] = v[q] * li * act_bwd(gt, p.act, p.alpha, p.gelu_tanh) * mg;
                dl[q] = v[q] * act_fwd(gt, p.act, p.alpha, p.gelu_tanh) * ml;
              }
              S* D = reinterpret_cast<S*>(p.c) + (size_t)row * p.ldc;
              store4(D + pg, dg);
              store4(D + pl, dl);
            }
          } else if constexpr (EPI == EPI_SRELU_FWD) {
            if (col < p.N) {
              if (p.bias) {
                const float* bb = p.bias + (size_t)e * p.ld_bias + col;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] += bb[q];
              }
              if (p.aux) store4(reinterpret_cast<S*>(p.aux) + (size_t)row * p.ld_aux + col, v);
              float o[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float hv = p.clamp > 0.0f ? fminf(v[q], p.clamp) : v[q];
                float r = fmaxf(hv, 0.0f);
                o[q] = r * r;
              }
              store4(reinterpret_cast<S*>(p.c) + (size_t)row * p.ldc + col, o);
            }
          } else if constexpr (EPI == EPI_SRELU_BWD) {
            if (col < p.N) {
              float hv[4], o[4];
              load4(reinterpret_cast<const S*>(p.aux) + (size_t)row * p.ld_aux + col, hv);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float hq = hv[q], m = 1.0f;
                if (p.clamp > 0.0f) {
                  m = hq <= p.clamp ? 1.0f : 0.0f;
                  hq = fminf(hq, p.clamp);
                }
                o[q] = v[q] * 2.0f * fmaxf(hq, 0.0f) * m;
              }
              store4(reinterpret_cast<S*>(p.c) + (size_t)row * p.ldc + col, o);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launching

template <class EL, bool AKM, bool BKM, int GROUP, int EPI, int BM, int BN, int WGM, int WGN>
moe_status_t launch_gemm(const GemmArgs& p, int max_cus, hipStream_t s) {
  typedef GemmCfg<EL, AKM, BKM, GROUP, EPI, BM, BN, WGM, WGN> C;
  auto kern = grouped_gemm_kernel<EL, AKM, BKM, GROUP, EPI, BM, BN, WGM, WGN>;
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

// Tile shapes: large problems take 256 x 256 tiles (4 waves of 128 x 128),
// small or narrow ones 128 x 128 (4 waves of 64 x 64).  fp32 takes 64 x 128.
template <class EL, bool AKM, bool BKM, int GROUP, int EPI>
moe_status_t dispatch_tiles(const GemmArgs& p, bool big, int max_cus, hipStream_t s) {
  if constexpr (sizeof(typename EL::storage) == 4) {
    return launch_gemm<EL, AKM, BKM, GROUP, EPI, 64, 128, 2, 2>(p, max_cus, s);
  } else {
    if (big) return launch_gemm<EL, AKM, BKM, GROUP, EPI, 256, 256, 2, 2>(p, max_cus, s);
    return launch_gemm<EL, AKM, BKM, GROUP, EPI, 128, 128, 2, 2>(p, max_cus, s);
  }
}

template <bool AKM, bool BKM, int GROUP, int EPI>
moe_status_t dispatch(int dtype, const GemmArgs& p, bool big, int max_cus, hipStream_t s) {
  if (dtype == MOE_BF16) return dispatch_tiles<BF16, AKM, BKM, GROUP, EPI>(p, big, max_cus, s);
  return dispatch_tiles<F32, AKM, BKM, GROUP, EPI>(p, big, max_cus, s);
}

inline GemmArgs zero_args() {
  GemmArgs p;
  memset(&p, 0, sizeof(p));
  p.alpha = 1.0f;
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

extern "C" {

moe_status_t moe_grouped_gemm_glu_fwd(const moe_glu_fwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= sizeof(moe_glu_fwd_args_t));
  MOE_CHECK_ARG(valid_dtype(a->dtype) && a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->d > 0 && a->f > 0 && a->d % 32 == 0 && a->f % 32 == 0);
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU || a->act == MOE_ACT_SRELU);
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool big = big_ragged_m(a->R, a->E, n1);
  if (gated) return dispatch<true, true, RAGGED_M, EPI_GLU_FWD>(a->dtype, p, big, a->max_cus, s);
  return dispatch<true, true, RAGGED_M, EPI_SRELU_FWD>(a->dtype, p, big, a->max_cus, s);
}

moe_status_t moe_grouped_gemm_fwd(const moe_gemm_fwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= sizeof(moe_gemm_fwd_args_t));
  MOE_CHECK_ARG(valid_dtype(a->dtype) && a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->N > 0 && a->K > 0 && a->N % 8 == 0 && a->K % 8 == 0);
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
  MOE_CHECK_ARG(a && a->struct_size >= sizeof(moe_glu_bwd_args_t));
  MOE_CHECK_ARG(valid_dtype(a->dtype) && a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->d > 0 && a->f > 0 && a->d % 32 == 0 && a->f % 32 == 0);
  MOE_CHECK_ARG(a->act == MOE_ACT_SWIGLU || a->act == MOE_ACT_GEGLU || a->act == MOE_ACT_SRELU);
  if (a->R == 0) return MOE_OK;
  MOE_CHECK_ARG(a->dy && a->w2 && a->h && a->offsets && a->dh);
  MOE_CHECK_ARG(aligned16(a->dy) && aligned16(a->w2) && aligned16(a->h) && aligned16(a->dh));
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool big = big_ragged_m(a->R, a->E, a->f);
  if (gated) return dispatch<true, false, RAGGED_M, EPI_GLU_BWD>(a->dtype, p, big, a->max_cus, s);
  return dispatch<true, false, RAGGED_M, EPI_SRELU_BWD>(a->dtype, p, big, a->max_cus, s);
}

moe_status_t moe_grouped_gemm_bwd(const moe_gemm_bwd_args_t* a, void* stream) {
  MOE_CHECK_ARG(a && a->struct_size >= sizeof(moe_gemm_bwd_args_t));
  MOE_CHECK_ARG(valid_dtype(a->dtype) && a->E >= 1 && a->E <= MOE_MAX_EXPERTS && a->R >= 0);
  MOE_CHECK_ARG(a->N > 0 && a->K > 0 && a->N % 8 == 0 && a->K % 8 == 0);
  MOE_CHECK_ARG(a->mode == MOE_BWD_DGRAD || a->mode == MOE_BWD_WGRAD);
  MOE_CHECK_ARG(a->g && a->offsets && a->out && aligned16(a->g) && aligned16(a->out));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemmArgs p = zero_args();
  p.offsets = a->offsets;
  p.E = a->E;
  p.R = a->R;
  if (a->mode == MOE_BWD_DGRAD) {
    if (a->R == 0) return MOE_OK;
    MOE_CHECK_ARG(a->w && aligned16(a->w));
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
  moe_status_t st = dispatch<false, false, RAGGED_K, EPI_STORE>(
      a->dtype, p, big_ragged_k(a->R, a->E, a->N, a->K), a->max_cus, s);
  if (st != MOE_OK || !a->db) return st;
  return launch_segment_colsum(a->dtype, a->g, a->offsets, a->E, a->R, a->N, a->db, s);
}

}  // extern "C"
