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
// Small batches (T*k <= kSmallPairs) run everything in one wavefront: one
// launch.  Larger batches use three kernels: per-chunk histograms, one
// block that scans them (and writes offsets and tiles), and per-chunk scatters.
#include "common.h"

namespace fp4moe {

constexpr int kSmallPairs = 1024;
constexpr int kChunk = 1024;       // pairs per chunk in the large path
constexpr int kMaxExperts = 4096;  // E + n_shared
constexpr int kIdBits = 13;        // ids < 8192 (two sentinel ids above kMaxExperts)
constexpr int kDroppedKey = 8191;
constexpr int kIdleKey = 8190;

__device__ __forceinline__ int pair_expert(const int32_t* ids, int p, int k, int topk, int E,
                                           bool* valid) {
  const int t = p / k, j = p - t * k;
  if (j < topk) {
    const int e = ids[(int64_t)t * topk + j];
    *valid = (e >= 0 && e < E);
    return e;
  }
  *valid = true;
  return E + (j - topk);
}

// Lanes holding the same key as this lane (wavefront match by bit ballots).
__device__ __forceinline__ uint64_t match_peers(int key) {
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// One 64-pair group of the stable scatter.  `cur` holds each expert's next
// sorted position (LDS) and is advanced by the lowest lane of each peer set.
__device__ __forceinline__ void scatter_group(const int32_t* ids, int p0, int P, int k, int topk,
                                              int E, int* cur, int32_t* sorted_pairs,
                                              int32_t* pair_pos) {
  const int lane = threadIdx.x & 63;
  const int p = p0 + lane;
  bool valid = false;
  int e = -1;
  if (p < P) e = pair_expert(ids, p, k, topk, E, &valid);
  const int key = (p >= P) ? kIdleKey : (valid ? e : kDroppedKey);
  const uint64_t peers = match_peers(key);
  const uint64_t lower = peers & ((1ull << lane) - 1ull);
  const int rank = __popcll(lower);
  const int leader = __ffsll((unsigned long long)peers) - 1;
  int base = 0;
  if (valid && lane == leader) {
    base = cur[e];
    cur[e] = base + __popcll(peers);
  }
  base = __shfl(base, leader, 64);
  if (p < P) {
    if (valid) {
      const int pos = base + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    } else {
      pair_pos[p] = -1;
    }
  }
}

// Exclusive scan of n values in LDS (in place) by one block of `nthreads`
// threads; returns the total to every thread.  Each thread owns a contiguous
// run; run sums are scanned through `tmp` (nthreads entries).
__device__ int block_exclusive_scan(int* vals, int n, int* tmp) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += vals[i];
  tmp[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the run sums.
  for (int off = 1; off < nt; off <<= 1) {
    const int v = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  const int total = tmp[nt - 1];
  int run = tmp[tid] - s;
  for (int i = lo; i < hi; ++i) {
    const int v = vals[i];
    vals[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Offsets, tiles and counters from the per-expert counts held in LDS `cnt`
// (overwritten with exclusive offsets).  `tcnt` receives tile offsets.
__device__ void finish_offsets(int* cnt, int* tcnt, int* tmp, int Et, int P, int block_m,
                               int32_t* expert_offsets, int32_t* tiles, int32_t* n_tiles,
                               int32_t* n_dropped, int32_t* sorted_pairs) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < Et; e += nt) tcnt[e] = (cnt[e] + block_m - 1) / block_m;
  __syncthreads();
  const int n_valid = block_exclusive_scan(cnt, Et, tmp);
  const int total_tiles = block_exclusive_scan(tcnt, Et, tmp);
  for (int e = tid; e < Et; e += nt) {
    expert_offsets[e] = cnt[e];
    const int c = ((e + 1 < Et) ? cnt[e + 1] : n_valid) - cnt[e];
    const int nte = (c + block_m - 1) / block_m;
    for (int m = 0; m < nte; ++m) {
      tiles[2 * (tcnt[e] + m)] = e;
      tiles[2 * (tcnt[e] + m) + 1] = m;
    }
  }
  for (int i = n_valid + tid; i < P; i += nt) sorted_pairs[i] = -1;
  if (tid == 0) {
    expert_offsets[Et] = n_valid;
    *n_tiles = total_tiles;
    *n_dropped = P - n_valid;
  }
}

// ---- small path: everything in one wavefront ------------------------------

__global__ __launch_bounds__(64) void permute_small_kernel(
    const int32_t* __restrict__ ids, int T, int topk, int E, int n_shared, int block_m,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int tcnt[kMaxExperts + 1];
  __shared__ int tmp[64];
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  const int lane = threadIdx.x;
  for (int e = lane; e < Et; e += 64) cnt[e] = 0;
  __syncthreads();
  for (int p = lane; p < P; p += 64) {
    bool valid;
    const int e = pair_expert(ids, p, k, topk, E, &valid);
    if (valid) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  finish_offsets(cnt, tcnt, tmp, Et, P, block_m, expert_offsets, tiles, n_tiles, n_dropped,
                 sorted_pairs);
  // cnt now holds each expert's first sorted position: the running cursor.
  for (int p0 = 0; p0 < P; p0 += 64) {
    scatter_group(ids, p0, P, k, topk, E, cnt, sorted_pairs, pair_pos);
    __syncthreads();
  }
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
  for (int e = threadIdx.x; e < Et; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = ws[(int64_t)b * Et + e];
      ws[(int64_t)b * Et + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  finish_offsets(cnt, tcnt, tmp, Et, P, block_m, expert_offsets, tiles, n_tiles, n_dropped,
                 sorted_pairs);
  for (int e = threadIdx.x; e < Et; e += blockDim.x) {
    const int off = cnt[e];
    for (int b = 0; b < nblk; ++b) ws[(int64_t)b * Et + e] += off;
  }
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int topk, int E, int n_shared,
    const int32_t* __restrict__ ws, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos) {
  __shared__ int cur[kMaxExperts];
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  const int32_t* base = ws + (int64_t)blockIdx.x * Et;
  for (int e = threadIdx.x; e < Et; e += 64) cur[e] = base[e];
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

extern "C" int moe_permute(const int32_t* topk_ids, int T, int topk, int E, int n_shared,
                           int block_m, void* workspace, size_t workspace_bytes,
                           int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                           int32_t* tiles, int32_t* n_tiles, int32_t* n_dropped, void* stream) {
  FP4MOE_REQUIRE(T >= 0, "moe_permute: T=%d < 0", T);
  FP4MOE_REQUIRE(topk >= 1 && topk <= 32, "moe_permute: topk=%d outside [1,32]", topk);
  FP4MOE_REQUIRE(n_shared >= 0 && n_shared <= 8, "moe_permute: n_shared=%d outside [0,8]",
                 n_shared);
  FP4MOE_REQUIRE(E >= 0 && E + n_shared >= 1 && E + n_shared <= kMaxExperts,
                 "moe_permute: E+n_shared=%d outside [1,%d]", E + n_shared, kMaxExperts);
  FP4MOE_REQUIRE(block_m >= 1 && block_m <= 1024, "moe_permute: block_m=%d", block_m);
  const int64_t P = (int64_t)T * (topk + n_shared);
  FP4MOE_REQUIRE(P < (1ll << 30), "moe_permute: too many pairs");
  FP4MOE_REQUIRE(expert_offsets && n_tiles && n_dropped && (T == 0 || tiles),
                 "moe_permute: null output pointer");
  FP4MOE_REQUIRE(T == 0 || (topk_ids && sorted_pairs && pair_pos), "moe_permute: null pointer");
  FP4MOE_CHECK_DEVICE();
  hipStream_t s = as_stream(stream);
  if (P <= kSmallPairs) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(64), 0, s, topk_ids, T, topk, E,
                       n_shared, block_m, expert_offsets, sorted_pairs, pair_pos, tiles, n_tiles,
                       n_dropped);
    return check_launch("moe_permute");
  }
  const size_t need = moe_permute_workspace(T, topk, E, n_shared, block_m);
  if (!workspace || workspace_bytes < need)
    return set_error(FP4MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu bytes",
                     workspace_bytes, need);
  const int nblk = (int)((P + kChunk - 1) / kChunk);
  int32_t* ws = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(256), 0, s, topk_ids, T, topk, E,
                     n_shared, ws);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, nblk, T, topk, E, n_shared,
                     block_m, ws, expert_offsets, sorted_pairs, tiles, n_tiles, n_dropped);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(64), 0, s, topk_ids, T, topk, E,
                     n_shared, ws, sorted_pairs, pair_pos);
  return check_launch("moe_permute");
}
