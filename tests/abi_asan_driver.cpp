// Host-side argument handling of the C ABI (include/moe.h) under
// AddressSanitizer, with no GPU: every entry point is called with bad
// arguments and must return the documented status code before touching the
// device, and every argument struct is passed at every size from 8 bytes to
// its full size, allocated on the heap at exactly that size -- so a read of a
// field past struct_size (the versioning rule of the ABI) is a
// heap-buffer-overflow that aborts this program.
//
// Built and run by tests/test_abi_asan.py against a host-only ASan build of
// the library sources.
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "moe.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);              \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

// 16-byte aligned addresses that are never dereferenced on the host
static void* const P = reinterpret_cast<void*>(0x10000);
static int32_t* const PI = reinterpret_cast<int32_t*>(0x20000);
static float* const PF = reinterpret_cast<float*>(0x30000);

static bool known(moe_status_t s) {
  return s == MOE_OK || s == MOE_ERR_INVALID_ARG || s == MOE_ERR_UNSUPPORTED ||
         s == MOE_ERR_WORKSPACE || s == MOE_ERR_HIP;
}

// Call fn with a copy of `full` cut to n bytes (struct_size = n) on the heap.
template <class A>
static moe_status_t call_cut(moe_status_t (*fn)(const A*, void*), const A& full, size_t n) {
  char* p = static_cast<char*>(std::malloc(n));
  std::memcpy(p, &full, n);
  size_t sz = n;
  std::memcpy(p, &sz, sizeof sz);
  moe_status_t st = fn(reinterpret_cast<const A*>(p), nullptr);
  std::free(p);
  return st;
}

template <class A>
static void sweep(const char* what, moe_status_t (*fn)(const A*, void*), const A& full,
                  size_t min_ok) {
  for (size_t n = sizeof(size_t); n <= sizeof(A); n += 4) {
    moe_status_t st = call_cut(fn, full, n);
    if (!known(st)) {
      std::printf("FAIL %s size %zu: unknown status %d\n", what, n, (int)st);
      ++g_fail;
    }
    // below the first size the entry point accepts it must refuse the struct
    if (n < min_ok && st != MOE_ERR_INVALID_ARG) {
      std::printf("FAIL %s size %zu accepted (status %d)\n", what, n, (int)st);
      ++g_fail;
    }
  }
}

// The harness's own check: a struct allocated short of the size it claims
// must be caught (the library then reads fields that are not there).
static int overread() {
  moe_gemm_fwd_args_t ff{};
  ff.struct_size = sizeof ff;            // claims every field ...
  ff.dtype = MOE_BF16; ff.a = P; ff.w = P; ff.offsets = PI; ff.E = 4; ff.R = 0; ff.N = 64;
  ff.K = 64; ff.y = P;
  const size_t n = offsetof(moe_gemm_fwd_args_t, a_mx);
  char* p = static_cast<char*>(std::malloc(n));   // ... but holds only the first version
  std::memcpy(p, &ff, n);
  moe_status_t st = moe_grouped_gemm_fwd(reinterpret_cast<const moe_gemm_fwd_args_t*>(p), nullptr);
  std::free(p);
  std::printf("over-read not caught (status %d)\n", (int)st);
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--overread") == 0) return overread();
  // ---- scalar queries
  EXPECT(std::strstr(moe_version(), "gfx950") != nullptr);
  EXPECT(std::strcmp(moe_status_string(MOE_OK), "MOE_OK") == 0);
  EXPECT(moe_status_string((moe_status_t)99) != nullptr);
  EXPECT(moe_glu_granularity() == 32);
  EXPECT(moe_permute_workspace_size(0, 8, 2) == 256);
  EXPECT(moe_permute_workspace_size(16384, 32, 8) % 256 == 0);
  EXPECT(moe_mx_col_len(100, 4) % 128 == 0 && moe_mx_col_len(100, 4) >= 100 + 31 * 4);
  EXPECT(moe_mx_col_ld(100, 4, MOE_BF16) == 0);

  // ---- routing
  EXPECT(moe_route_topk(nullptr, 4, 8, 2, 0, 1, PI, PF, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(PF, 4, 2, 3, 0, 1, PI, PF, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(PF, 4, 8, 2, 7, 1, PI, PF, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(PF, 4, 2000, 2, 0, 1, PI, PF, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(nullptr, 0, 8, 2, 0, 1, nullptr, nullptr, nullptr, nullptr) == MOE_OK);
  EXPECT(moe_route_topk_bwd(PF, nullptr, PF, 4, 8, 2, 0, 1, PF, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk_bwd(PF, PI, PF, 4, 8, 9, 0, 1, PF, nullptr) == MOE_ERR_INVALID_ARG);

  // ---- fused router
  EXPECT(moe_router_topk(P, P, MOE_F32, 4, 64, 8, 2, 0, 1, PF, PI, PF, nullptr, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_router_topk(P, P, 9, 4, 64, 8, 2, 0, 1, PF, PI, PF, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_router_topk(P, P, MOE_BF16, 4, 48, 8, 2, 0, 1, PF, PI, PF, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);                                                   // d % 32
  EXPECT(moe_router_topk(P, P, MOE_BF16, 4, 64, 8, 2, 0, 1, PF, PI, nullptr, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);                                                   // idx without w
  EXPECT(moe_router_topk(P, P, MOE_BF16, 4, 64, 300, 2, 0, 1, nullptr, PI, PF, nullptr,
                         nullptr) == MOE_ERR_INVALID_ARG);                       // E > 256: logits
  EXPECT(moe_router_topk(P, P, MOE_BF16, 4, 64, 8, 9, 0, 1, PF, PI, PF, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);                                                   // k > E
  EXPECT(moe_router_topk(nullptr, nullptr, MOE_BF16, 0, 64, 8, 2, 0, 1, PF, PI, PF, nullptr,
                         nullptr) == MOE_OK);
  EXPECT(moe_router_bwd(P, P, MOE_BF16, PF, 4, 40, 8, PF, 0, P, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_router_bwd(P, P, MOE_BF16, PF, 4, (1 << 20) + 32, 8, PF, 0, P, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_router_bwd(nullptr, P, MOE_BF16, PF, 4, 64, 8, PF, 0, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);                                                   // dWr without x
  EXPECT(moe_router_bwd(P, P, MOE_F32, PF, 4, 64, 8, PF, 0, P, nullptr) == MOE_ERR_UNSUPPORTED);

  // ---- permute (with and without a workspace)
  EXPECT(moe_permute(nullptr, MOE_BF16, 1000, 0, PI, 2, 8, PI, PI, nullptr, PI, PI, nullptr, P, 4,
                     nullptr, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_permute(nullptr, MOE_BF16, 1000, 0, PI, 2, 8, PI, PI, nullptr, PI, PI, nullptr,
                     nullptr, 4096, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute(nullptr, MOE_BF16, 10, 64, PI, 2, 8, PI, PI, nullptr, PI, PI, P, P, 4096,
                     nullptr, nullptr) == MOE_ERR_INVALID_ARG);                 // xp without x
  EXPECT(moe_permute(P, MOE_BF16, 10, 60, PI, 2, 8, PI, PI, nullptr, PI, PI, P, P, 4096, nullptr,
                     nullptr) == MOE_ERR_INVALID_ARG);                          // row not 16 bytes
  EXPECT(moe_permute(nullptr, MOE_BF16, 10, 0, PI, 9, 8, PI, PI, nullptr, PI, PI, nullptr, P,
                     4096, nullptr, nullptr) == MOE_ERR_INVALID_ARG);           // k > E
  EXPECT(moe_permute_noalloc(nullptr, MOE_BF16, 1025 * 128, 0, PI, 8, 256, PI, PI, nullptr, PI, PI,
                             nullptr, nullptr, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_permute_noalloc(nullptr, MOE_BF16, 100, 0, PI, 8, 2000, PI, PI, nullptr, PI, PI,
                             nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);

  // ---- repack / transpose
  EXPECT(moe_repack_glu_weights(P, nullptr, MOE_BF16, 2, 48, 64, 0, P, nullptr, nullptr) ==
         MOE_ERR_INVALID_ARG);                                                   // f % 32
  EXPECT(moe_transpose_weights(P, MOE_BF16, 2, 12, 64, P, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_transpose_weights(P, MOE_BF16, 2, 64, 64, P, nullptr) == MOE_ERR_INVALID_ARG);  // alias

  // ---- combine
  EXPECT(moe_unpermute_combine(nullptr, MOE_BF16, PI, PF, 4, 2, 64, P, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_unpermute_combine(P, 9, PI, PF, 4, 2, 64, P, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_unpermute_combine(P, MOE_BF16, PI, PF, 4, 2, 60, P, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_unpermute_combine_bwd(P, P, MOE_BF16, nullptr, PF, 4, 2, 64, P, PF, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_unpermute_combine_bwd(P, nullptr, MOE_BF16, PI, nullptr, 4, 2, 64, P, PF, nullptr) ==
         MOE_ERR_INVALID_ARG);                          // a gate gradient needs y
  moe_mx_t mx{static_cast<uint8_t*>(P), static_cast<uint8_t*>(P), 60};
  EXPECT(moe_unpermute_combine_mx(&mx, MOE_E4M3, PI, PF, 4, 2, 64, P, MOE_BF16, nullptr) ==
         MOE_ERR_INVALID_ARG);

  // ---- MX quantizers
  EXPECT(moe_mx_quantize(P, MOE_BF16, 4, 48, &mx, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_mx_quantize(P, MOE_BF16, 4, 64, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_mxfp4_quantize(P, MOE_BF16, 4, 48, &mx, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_mx_quantize_transpose(P, MOE_BF16, 2, 30, 64, &mx, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_mxfp4_quantize_transpose(P, MOE_BF16, 2, 30, 64, &mx, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_mx_quantize_experts(P, MOE_BF16, PI, PI, nullptr, 2, PI, PI, 4, 64, 64, &mx, nullptr,
                                 nullptr) == MOE_ERR_INVALID_ARG);   // row_map without topk_w
  EXPECT(moe_mxfp4_quantize_experts(P, MOE_BF16, PI, PI, nullptr, 2, PI, PI, 4, 64, 64, &mx,
                                    nullptr, nullptr) == MOE_ERR_INVALID_ARG);

  // ---- grouped GEMM argument structs: every prefix size (R = 0: nothing to launch)
  moe_glu_fwd_args_t gf{};
  gf.dtype = MOE_BF16; gf.xp = P; gf.w1p = P; gf.offsets = PI; gf.E = 4; gf.R = 0; gf.d = 64;
  gf.f = 64; gf.act = MOE_ACT_SWIGLU; gf.alpha = 1.0f; gf.a_out = P; gf.src_row = PI;
  sweep("glu_fwd", moe_grouped_gemm_glu_fwd, gf, offsetof(moe_glu_fwd_args_t, xp_mx));
  moe_gemm_fwd_args_t ff{};
  ff.dtype = MOE_BF16; ff.a = P; ff.w = P; ff.offsets = PI; ff.E = 4; ff.R = 0; ff.N = 64;
  ff.K = 64; ff.y = P;
  sweep("gemm_fwd", moe_grouped_gemm_fwd, ff, offsetof(moe_gemm_fwd_args_t, a_mx));
  moe_glu_bwd_args_t gb{};
  gb.dtype = MOE_BF16; gb.dy = P; gb.w2 = P; gb.h = P; gb.offsets = PI; gb.E = 4; gb.R = 0;
  gb.d = 64; gb.f = 64; gb.act = MOE_ACT_SWIGLU; gb.alpha = 1.0f; gb.dh = P; gb.w2t = P;
  sweep("glu_bwd", moe_grouped_gemm_glu_bwd, gb, offsetof(moe_glu_bwd_args_t, dy_mx));
  moe_gemm_bwd_args_t bb{};
  bb.dtype = MOE_BF16; bb.mode = MOE_BWD_DGRAD; bb.g = P; bb.w = P; bb.offsets = PI; bb.E = 4;
  bb.R = 0; bb.N = 64; bb.K = 64; bb.out = P; bb.wt = P;
  sweep("gemm_bwd dgrad", moe_grouped_gemm_bwd, bb, offsetof(moe_gemm_bwd_args_t, g_mx));
  // the same structs with an argument error that is only found in a field past
  // the first version: refused whenever the struct holds it
  moe_gemm_fwd_args_t ff2 = ff;
  ff2.y_mx = &mx;                 // an MX output for bf16 operands
  EXPECT(call_cut(moe_grouped_gemm_fwd, ff2, sizeof ff2) == MOE_ERR_INVALID_ARG);
  moe_gemm_bwd_args_t bb2 = bb;
  bb2.a_src_row = PI;             // a gather index for a dgrad
  EXPECT(call_cut(moe_grouped_gemm_bwd, bb2, sizeof bb2) == MOE_ERR_INVALID_ARG);
  moe_gemm_bwd_args_t bw = bb;
  bw.mode = MOE_BWD_WGRAD; bw.a = P; bw.R = 8; bw.a_src_row = PI; bw.a_src_rows = 0;
  EXPECT(call_cut(moe_grouped_gemm_bwd, bw, sizeof bw) == MOE_ERR_INVALID_ARG);  // no rows to gather
  moe_glu_fwd_args_t gf2 = gf;
  gf2.dtype = MOE_E4M3; gf2.xp_mx = &mx; gf2.w1_mx = &mx; gf2.R = 8;
  EXPECT(call_cut(moe_grouped_gemm_glu_fwd, gf2, sizeof gf2) == MOE_ERR_INVALID_ARG);  // src_row + MX
  moe_glu_bwd_args_t gb2 = gb;
  gb2.act = 7;
  EXPECT(call_cut(moe_grouped_gemm_glu_bwd, gb2, sizeof gb2) == MOE_ERR_INVALID_ARG);
  // feature-scaling gradient without (or with too small) a workspace: refused
  // before anything is enqueued
  moe_glu_bwd_args_t gb3 = gb;
  gb3.R = 8; gb3.row_scale = PF; gb3.d_row_scale = PF;
  EXPECT(call_cut(moe_grouped_gemm_glu_bwd, gb3, sizeof gb3) == MOE_ERR_WORKSPACE);
  gb3.ws = P; gb3.ws_bytes = moe_glu_bwd_workspace_size(8, 64) - 4;
  EXPECT(call_cut(moe_grouped_gemm_glu_bwd, gb3, sizeof gb3) == MOE_ERR_WORKSPACE);
  EXPECT(moe_glu_bwd_workspace_size(8, 64) == 2 * 8 * sizeof(float));
  EXPECT(moe_glu_bwd_workspace_size(0, 64) == 0);

  // ---- gates to and from row order
  EXPECT(moe_permute_rows(PF, PI, -1, 0, PF + 64, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute_rows(PF, PI, 8, 2, PF + 64, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute_rows(PF, PI, 8, 0, PF, nullptr) == MOE_ERR_INVALID_ARG);   // in place
  EXPECT(moe_permute_rows(nullptr, PI, 8, 1, PF, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute_rows(nullptr, nullptr, 0, 0, nullptr, nullptr) == MOE_OK);

  if (g_fail == 0) std::printf("abi host checks passed\n");
  return g_fail == 0 ? 0 : 1;
}
