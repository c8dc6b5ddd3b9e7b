// moe_permute: stable sort of (token, slot) pairs by expert, plus the tile list.
//
// [NVFP4] "Memory Management": only dispatched experts are touched.
// [GAUDI] "What it taught about Gaudi": cost must follow the routing, empty
// expert slots are skipped.  [K3]: expert tiles carry padding rows.
//
// Stability without atomics in the scatter: pairs are visited in ascending p
// by a single wavefront per chunk; within a 64-pair group the lanes that share
// an expert are found with one ballot per id bit (a wavefront "match"), their
// rank is the popcount of lower peer lanes, and the lowest peer advances the
// expert's running position in LDS.
//
// Small batches (T*k <= kSmallPairs) take one launch: with at most
// kHistMaxExperts experts, one wavefront per 64 pairs and per-group
// histograms (permute_hist_body); with more experts, one wavefront that
// visits the groups in order.  Larger batches use three kernels: per-chunk histograms, one
// block that scans them (and writes offsets and tiles), and per-chunk scatters.
#include <mutex>

#include "permute_dev.h"

namespace fp4moe {

// ---- the library-owned chunk-histogram buffer of moe_permute_noalloc -------
//
// A file-scope device array: every GPU the library runs on holds its own copy
// (in this file's code object) until the process ends.  Host code never
// passes the array's name to a kernel -- on the host that name is only a
// stand-in -- but the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch_ptr.
// The large path writes every (chunk, expert) count before reading it, so the
// buffer needs no clearing between calls.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;   // 4 MiB
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return set_error(FP4MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: no current HIP device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(FP4MOE_ERR_LAUNCH, "moe_permute_noalloc: hipGetSymbolAddress on device "
                       "%d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP4MOE_OK;
}

// ---- small path: everything in one wavefront ------------------------------

__global__ __launch_bounds__(64) void permute_small_kernel(
    const int32_t* __restrict__ ids, int T, int topk, int E, int n_shared, int block_m,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped) {
  __shared__ PermuteSmallScratch lds;
  permute_small_body(ids, T, topk, E, n_shared, block_m, expert_offsets, sorted_pairs, pair_pos,
                     tiles, n_tiles, n_dropped, lds);
}

__global__ __launch_bounds__(1024) void permute_small_hist_kernel(
    const int32_t* __restrict__ ids, int T, int topk, int E, int n_shared, int block_m,
    int max_tiles, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped) {
  __shared__ PermuteHistScratch lds;
  permute_hist_body(ids, T, topk, E, n_shared, block_m, max_tiles, expert_offsets, sorted_pairs,
                    pair_pos, tiles, n_tiles, n_dropped, lds);
}

// ---- large path ------------------------------------------------------------

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids,
                                                           int T, int topk, int E, int n_shared,
                                                           int32_t* __restrict__ ws) {
  __shared__ int cnt[kMaxExperts];
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  for (int e = threadIdx.x; e < Et; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kChunk, p1 = min(P, p0 + kChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    bool valid;
    const int e = pair_expert(ids, p, k, topk, E, &valid);
    if (valid) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int32_t* out = ws + (int64_t)blockIdx.x * Et;
  for (int e = threadIdx.x; e < Et; e += blockDim.x) out[e] = cnt[e];
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(
    int nblk, int T, int topk, int E, int n_shared, int block_m, int32_t* __restrict__ ws,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, int32_t* __restrict__ n_dropped) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int tcnt[kMaxExperts + 1];
  __shared__ int tmp[1024];
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  // Per expert: exclusive scan over the chunks (in place), total into cnt.
  // The counts are loaded kScanBatch at a time, so that one memory round trip
  // serves kScanBatch chunks instead of one.
  constexpr int kScanBatch = 16;
  for (int e = threadIdx.x; e < Et; e += blockDim.x) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j)
        c[j] = (b0 + j < nblk) ? ws[(int64_t)(b0 + j) * Et + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) ws[(int64_t)(b0 + j) * Et + e] = run;
        run += c[j];
      }
    }
    cnt[e] = run;
  }
  __syncthreads();
  // expert_offsets receives each expert's first sorted position; the scatter
  // adds it to the chunk prefixes left in ws
  finish_offsets(cnt, tcnt, tmp, Et, P, block_m, expert_offsets, tiles, n_tiles, n_dropped,
                 sorted_pairs);
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int topk, int E, int n_shared,
    const int32_t* __restrict__ ws, const int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
  __shared__ int cur[kMaxExperts];
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  // cursor = expert's first sorted position + pairs of the expert in earlier chunks
  const int32_t* base = ws + (int64_t)blockIdx.x * Et;
  for (int e = threadIdx.x; e < Et; e += 64) cur[e] = expert_offsets[e] + base[e];
  __syncthreads();
  const int p0 = blockIdx.x * kChunk, p1 = min(P, p0 + kChunk);
  for (int g = p0; g < p1; g += 64) {
    scatter_group(ids, g, p1, k, topk, E, cur, sorted_pairs, pair_pos);
    __syncthreads();
  }
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int moe_permute_max_tiles(int T, int topk, int E, int n_shared, int block_m) {
  if (T < 0 || topk < 1 || n_shared < 0 || E < 0 || block_m < 1) return 0;
  const int64_t P = (int64_t)T * (topk + n_shared);
  const int64_t ne = (E + n_shared) < P ? (E + n_shared) : P;
  return (int)((P + ne * (block_m - 1)) / block_m);
}

extern "C" size_t moe_permute_workspace(int T, int topk, int E, int n_shared, int block_m) {
  (void)block_m;
  const int64_t P = (int64_t)T * (topk + n_shared);
  if (P <= kSmallPairs) return 0;
  const int64_t nblk = (P + kChunk - 1) / kChunk;
  return (size_t)(nblk * (E + n_shared) * sizeof(int32_t));
}

// Argument checks shared by moe_permute and moe_permute_noalloc.
static int permute_check(const char* who, const int32_t* topk_ids, int T, int topk, int E,
                         int n_shared, int block_m, int32_t* expert_offsets, int32_t* sorted_pairs,
                         int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles, int32_t* n_dropped) {
  FP4MOE_REQUIRE(T >= 0, "%s: T=%d < 0", who, T);
  FP4MOE_REQUIRE(topk >= 1 && topk <= 32, "%s: topk=%d outside [1,32]", who, topk);
  FP4MOE_REQUIRE(n_shared >= 0 && n_shared <= 8, "%s: n_shared=%d outside [0,8]", who,
                 n_shared);
  FP4MOE_REQUIRE(E >= 0 && E + n_shared >= 1 && E + n_shared <= kMaxExperts,
                 "%s: E+n_shared=%d outside [1,%d]", who, E + n_shared, kMaxExperts);
  FP4MOE_REQUIRE(block_m >= 1 && block_m <= 1024, "%s: block_m=%d", who, block_m);
  const int64_t P = (int64_t)T * (topk + n_shared);
  FP4MOE_REQUIRE(P < (1ll << 30), "%s: too many pairs", who);
  FP4MOE_REQUIRE(expert_offsets && n_tiles && n_dropped && (T == 0 || tiles),
                 "%s: null output pointer", who);
  FP4MOE_REQUIRE(T == 0 || (topk_ids && sorted_pairs && pair_pos), "%s: null pointer", who);
  return FP4MOE_OK;
}

// The launches; ws holds moe_permute_workspace() bytes whenever the batch
// takes the large path.
static int permute_launch(const char* who, const int32_t* topk_ids, int T, int topk, int E,
                          int n_shared, int block_m, int32_t* ws, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, int32_t* tiles,
                          int32_t* n_tiles, int32_t* n_dropped, hipStream_t s) {
  const int64_t P = (int64_t)T * (topk + n_shared);
  if (P <= kSmallPairs && E + n_shared <= kHistMaxExperts) {
    const int nw = P > 64 ? (int)((P + 63) / 64) : 1;
    hipLaunchKernelGGL(permute_small_hist_kernel, dim3(1), dim3(64 * nw), 0, s, topk_ids, T, topk,
                       E, n_shared, block_m, moe_permute_max_tiles(T, topk, E, n_shared, block_m),
                       expert_offsets, sorted_pairs, pair_pos, tiles, n_tiles, n_dropped);
    return check_launch(who);
  }
  if (P <= kSmallPairs) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(64), 0, s, topk_ids, T, topk, E,
                       n_shared, block_m, expert_offsets, sorted_pairs, pair_pos, tiles, n_tiles,
                       n_dropped);
    return check_launch(who);
  }
  const int nblk = (int)((P + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(256), 0, s, topk_ids, T, topk, E,
                     n_shared, ws);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, nblk, T, topk, E, n_shared,
                     block_m, ws, expert_offsets, sorted_pairs, tiles, n_tiles, n_dropped);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(64), 0, s, topk_ids, T, topk, E,
                     n_shared, ws, expert_offsets, sorted_pairs, pair_pos);
  return check_launch(who);
}

extern "C" int moe_permute(const int32_t* topk_ids, int T, int topk, int E, int n_shared,
                           int block_m, void* workspace, size_t workspace_bytes,
                           int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                           int32_t* tiles, int32_t* n_tiles, int32_t* n_dropped, void* stream) {
  int st = permute_check("moe_permute", topk_ids, T, topk, E, n_shared, block_m, expert_offsets,
                         sorted_pairs, pair_pos, tiles, n_tiles, n_dropped);
  if (st != FP4MOE_OK) return st;
  const int64_t P = (int64_t)T * (topk + n_shared);
  const size_t need = moe_permute_workspace(T, topk, E, n_shared, block_m);
  if (P > kSmallPairs && (!workspace || workspace_bytes < need))
    return set_error(FP4MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu bytes",
                     workspace_bytes, need);
  FP4MOE_CHECK_DEVICE();
  return permute_launch("moe_permute", topk_ids, T, topk, E, n_shared, block_m,
                        static_cast<int32_t*>(workspace), expert_offsets, sorted_pairs, pair_pos,
                        tiles, n_tiles, n_dropped, as_stream(stream));
}

extern "C" size_t moe_permute_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

extern "C" int moe_permute_noalloc(const int32_t* topk_ids, int T, int topk, int E, int n_shared,
                                   int block_m, int32_t* expert_offsets, int32_t* sorted_pairs,
                                   int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles,
                                   int32_t* n_dropped, void* stream) {
  int st = permute_check("moe_permute_noalloc", topk_ids, T, topk, E, n_shared, block_m,
                         expert_offsets, sorted_pairs, pair_pos, tiles, n_tiles, n_dropped);
  if (st != FP4MOE_OK) return st;
  const size_t need = moe_permute_workspace(T, topk, E, n_shared, block_m);
  if (need > kNoAllocScratchBytes)
    return set_error(FP4MOE_ERR_WORKSPACE,
                     "moe_permute_noalloc: this batch needs %zu bytes of chunk histograms, more "
                     "than the library's %zu-byte buffer; call moe_permute with a workspace",
                     need, kNoAllocScratchBytes);
  FP4MOE_CHECK_DEVICE();
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != FP4MOE_OK) return st;
  }
  return permute_launch("moe_permute_noalloc", topk_ids, T, topk, E, n_shared, block_m,
                        static_cast<int32_t*>(ws), expert_offsets, sorted_pairs, pair_pos, tiles,
                        n_tiles, n_dropped, as_stream(stream));
}
