// Permute routed assignments into expert-contiguous rows, with the per-expert
// counts and offsets produced and kept in device memory.
//
// [P2] "JAXとNVIDIA Transformer EngineによるDropless MoE学習の高速化", section
// "主張と根拠": the rows of each expert form one ragged group whose size is
// known only at run time.  [P1] "高度な融合カーネルによる MoE 学習スループット
// の向上", section "ホストとデバイスの同期および CPU 起動オーバーヘッドの排除":
// the tokens per group are tracked in GPU memory, so nothing is read back.
//
// Row of assignment i = t*k + j with expert e:  offsets[e] + #{i' < i : e(i') = e}
// (a stable counting sort).  Four kernels, all sized from host-known T*k:
//   1. count:   per chunk of CHUNK assignments, a per-expert histogram
//               (integer LDS atomics: the result does not depend on order).
//   2. scan:    per expert, the exclusive prefix over chunks; counts; the
//               exclusive scan over experts -> offsets (and padded offsets).
//   3. scatter: per chunk, each assignment's rank among the earlier ones of
//               its expert, from wave ballots on the expert-id bits
//               (64 assignments per wave, waves in order), plus the chunk
//               base -> row_map, src_row.
//   4. gather:  xp[r] = x[src_row[r]], one wave per row, 16-byte vectors.
#include "common.hpp"

#include <mutex>

namespace moe {

static constexpr int PERM_THREADS = 256;
static constexpr int PERM_ITEMS = 4;  // assignments per thread per chunk
static constexpr int CHUNK = PERM_THREADS * PERM_ITEMS;

__device__ __forceinline__ int read_expert(const int32_t* idx, int i, int E, int32_t* err_word) {
  int e = idx[i];
  if (e < 0 || e >= E) {
    set_err(err_word, MOE_ERRBIT_BAD_EXPERT);
    e = 0;
  }
  return e;
}

__global__ void __launch_bounds__(PERM_THREADS) permute_count_kernel(
    const int32_t* __restrict__ idx, int n, int E, int32_t* __restrict__ chunk_counts,
    int32_t* err_word) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) hist[e] = 0;
  __syncthreads();
  int base = blockIdx.x * CHUNK;
  for (int it = 0; it < PERM_ITEMS; ++it) {
    int i = base + it * PERM_THREADS + threadIdx.x;
    if (i < n) atomicAdd(&hist[read_expert(idx, i, E, err_word)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS)
    chunk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads; thread e owns expert e.
__global__ void __launch_bounds__(1024) permute_scan_kernel(
    int32_t* __restrict__ chunk_counts, int nchunks, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pad_offsets) {
  __shared__ int32_t s_tot[1024];
  __shared__ int32_t s_pad[1024];
  int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      int32_t v = chunk_counts[(size_t)c * E + e];
      chunk_counts[(size_t)c * E + e] = tot;  // exclusive prefix within expert e
      tot += v;
    }
    counts[e] = tot;
  }
  s_tot[e] = (e < E) ? tot : 0;
  s_pad[e] = (e < E) ? (tot + 31) / 32 * 32 : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 slots.
  for (int o = 1; o < 1024; o <<= 1) {
    int a = (e >= o) ? s_tot[e - o] : 0;
    int b = (e >= o) ? s_pad[e - o] : 0;
    __syncthreads();
    s_tot[e] += a;
    s_pad[e] += b;
    __syncthreads();
  }
  int excl = s_tot[e] - ((e < E) ? tot : 0);
  if (e < E) {
    offsets[e] = excl;
    if (pad_offsets) pad_offsets[e] = s_pad[e] - (tot + 31) / 32 * 32;
    for (int c = 0; c < nchunks; ++c) chunk_counts[(size_t)c * E + e] += excl;
  }
  if (e == E - 1) {
    offsets[E] = s_tot[e];
    if (pad_offsets) pad_offsets[E] = s_pad[e];
  }
}

__global__ void __launch_bounds__(PERM_THREADS) permute_scatter_kernel(
    const int32_t* __restrict__ idx, int n, int k, int E,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ row_map,
    int32_t* __restrict__ src_row) {
  constexpr int NW = PERM_THREADS / 64;
  extern __shared__ int32_t sh[];
  int32_t* run = sh;            // [E]   next row of each expert
  int32_t* wcnt = sh + E;       // [NW][E] per-wave counts of the current round
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    run[e] = chunk_base[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < NW; ++w) wcnt[w * E + e] = 0;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = blockIdx.x * CHUNK;
  for (int it = 0; it < PERM_ITEMS; ++it) {
    int i = base + it * PERM_THREADS + threadIdx.x;
    bool valid = i < n;
    int e = 0;
    if (valid) {
      e = idx[i];
      if (e < 0 || e >= E) e = 0;  // flagged by the count kernel
    }
    // lanes of this wave holding the same expert
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      uint64_t bb = __ballot(valid && ((e >> b) & 1));
      match &= ((e >> b) & 1) ? bb : ~bb;
    }
    int rank = __popcll(match & lt_mask);
    bool leader = valid && rank == 0;
    if (leader) wcnt[wv * E + e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int r = run[e] + rank;
      for (int w = 0; w < wv; ++w) r += wcnt[w * E + e];
      row_map[i] = r;
      src_row[r] = i / k;
    }
    __syncthreads();
    for (int e2 = threadIdx.x; e2 < E; e2 += PERM_THREADS) {
      int add = 0;
      for (int w = 0; w < NW; ++w) {
        add += wcnt[w * E + e2];
        wcnt[w * E + e2] = 0;
      }
      run[e2] += add;
    }
    __syncthreads();
  }
}

// xp[r] = x[src_row[r]]; one wave per row, 16-byte chunks.
__global__ void __launch_bounds__(256) gather_rows_kernel(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ src_row,
                                                          int R, int T, int chunks_per_row,
                                                          u32x4* __restrict__ xp) {
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  int lane = threadIdx.x & 63;
  int t = src_row[r];
  t = (t < 0 || t >= T) ? 0 : t;
  const u32x4* src = x + (size_t)t * chunks_per_row;
  u32x4* dst = xp + (size_t)r * chunks_per_row;
  for (int c = lane; c < chunks_per_row; c += 64) dst[c] = src[c];
}

// The four kernels above on the caller's stream; ws holds the per-chunk,
// per-expert counts (every entry is written by the count kernel before it
// is read, so ws needs no clearing).
static moe_status_t permute_run(const void* x, int dtype, int T, int d, const int32_t* topk_idx, int k,
                         int E, int32_t* counts, int32_t* offsets, int32_t* pad_offsets,
                         int32_t* row_map, int32_t* src_row, void* xp, int32_t* chunk_counts,
                         int32_t* err_word, hipStream_t s) {
  const size_t n = (size_t)T * k;
  const int nchunks = (int)((n + CHUNK - 1) / CHUNK);
  if (nchunks > 0) {
    hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(PERM_THREADS),
                       E * sizeof(int32_t), s, topk_idx, (int)n, E, chunk_counts, err_word);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E,
                     counts, offsets, pad_offsets);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  if (nchunks > 0) {
    size_t shm = (size_t)E * (1 + PERM_THREADS / 64) * sizeof(int32_t);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(PERM_THREADS), shm, s,
                       topk_idx, (int)n, k, E, chunk_counts, row_map, src_row);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    if (xp) {
      int cpr = (int)(d * dtype_size(dtype) / 16);
      hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s,
                         reinterpret_cast<const u32x4*>(x), src_row, (int)n, T, cpr,
                         reinterpret_cast<u32x4*>(xp));
      if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    }
  }
  return MOE_OK;
}

// Argument checks shared by both entry points.
static moe_status_t permute_check(const void* x, int dtype, int T, int d, const int32_t* topk_idx,
                           int k, int E, int32_t* counts, int32_t* offsets, int32_t* row_map,
                           int32_t* src_row, void* xp) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= E);
  MOE_CHECK_ARG(counts && offsets);
  MOE_CHECK_ARG((size_t)T * k < (size_t)INT32_MAX);
  if (xp) {
    MOE_CHECK_ARG(x && valid_dtype(dtype) && d > 0);
    MOE_CHECK_ARG(aligned16(x) && aligned16(xp) && (d * dtype_size(dtype)) % 16 == 0);
  }
  if (T > 0) MOE_CHECK_ARG(topk_idx && row_map && src_row);
  return MOE_OK;
}

}  // namespace moe

// Scratch of the allocation-free permute (moe_permute_noalloc): the
// per-chunk, per-expert counts that moe_permute keeps in the caller's
// workspace.  Each device holds its own copy until the process ends; in host
// code `scratch` names only a host-side stand-in, so the device address is
// looked up once per device (hipGetSymbolAddress) and only that is used.
static constexpr size_t kPermuteScratchBytes = MOE_PERMUTE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) int32_t scratch[kPermuteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on its first use).
// A float per assignment to and from the expert-contiguous row order:
// forward dst[row_map[i]] = src[i], inverse dst[i] = src[row_map[i]];
// indices outside [0, n) are skipped (forward) or read as 0 (inverse).
__global__ void __launch_bounds__(256) permute_rows_kernel(const float* __restrict__ src,
                                                           const int32_t* __restrict__ row_map,
                                                           int n, int inverse,
                                                           float* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = row_map[i];
  const bool ok = r >= 0 && r < n;
  if (inverse)
    dst[i] = ok ? src[r] : 0.0f;
  else if (ok)
    dst[r] = src[i];
}

moe_status_t scratch_on_current_device(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return MOE_OK;
}
}  // namespace

using namespace moe;

extern "C" {

size_t moe_permute_workspace_size(int T, int E, int k) {
  if (T <= 0 || E <= 0 || k <= 0) return 256;
  size_t n = (size_t)T * k;
  size_t nchunks = (n + CHUNK - 1) / CHUNK;
  return (nchunks * (size_t)E * sizeof(int32_t) + 255) / 256 * 256;
}

moe_status_t moe_permute(const void* x, int dtype, int T, int d, const int32_t* topk_idx,
                         int k, int E, int32_t* counts, int32_t* offsets,
                         int32_t* pad_offsets, int32_t* row_map, int32_t* src_row, void* xp,
                         void* ws, size_t ws_bytes, int32_t* err_word, void* stream) {
  moe_status_t st =
      permute_check(x, dtype, T, d, topk_idx, k, E, counts, offsets, row_map, src_row, xp);
  if (st != MOE_OK) return st;
  if (T > 0) {
    MOE_CHECK_ARG(ws);
    if (ws_bytes < moe_permute_workspace_size(T, E, k)) return MOE_ERR_WORKSPACE;
  }
  return permute_run(x, dtype, T, d, topk_idx, k, E, counts, offsets, pad_offsets, row_map,
                     src_row, xp, reinterpret_cast<int32_t*>(ws), err_word,
                     reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_permute_noalloc(const void* x, int dtype, int T, int d,
                                 const int32_t* topk_idx, int k, int E, int32_t* counts,
                                 int32_t* offsets, int32_t* pad_offsets, int32_t* row_map,
                                 int32_t* src_row, void* xp, int32_t* err_word, void* stream) {
  moe_status_t st =
      permute_check(x, dtype, T, d, topk_idx, k, E, counts, offsets, row_map, src_row, xp);
  if (st != MOE_OK) return st;
  // sizes beyond the static scratch are refused before anything touches the device
  if (moe_permute_workspace_size(T, E, k) > kPermuteScratchBytes) return MOE_ERR_WORKSPACE;
  int32_t* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MOE_OK) return st;
  return permute_run(x, dtype, T, d, topk_idx, k, E, counts, offsets, pad_offsets, row_map,
                     src_row, xp, ws, err_word, reinterpret_cast<hipStream_t>(stream));
}

moe_status_t moe_permute_rows(const float* src, const int32_t* row_map, int n, int inverse,
                              float* dst, void* stream) {
  MOE_CHECK_ARG(n >= 0 && (inverse == 0 || inverse == 1));
  if (n == 0) return MOE_OK;
  MOE_CHECK_ARG(src && row_map && dst && src != dst);
  hipLaunchKernelGGL(permute_rows_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), src, row_map, n, inverse, dst);
  return launch_status();
}

}  // extern "C"
