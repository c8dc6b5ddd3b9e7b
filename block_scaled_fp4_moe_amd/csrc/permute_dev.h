// Device code of moe_permute, shared by the permutation kernels and the fused
// small-batch routing + permutation kernel.
#pragma once
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

struct PermuteSmallScratch {
  int cnt[kMaxExperts + 1];
  int tcnt[kMaxExperts + 1];
  int tmp[1024];
};

// The whole permutation of P <= kSmallPairs pairs by one block (any number of
// wavefronts; every thread of the block calls it).  ids may live in LDS.
__device__ __forceinline__ void permute_small_body(
    const int32_t* ids, int T, int topk, int E, int n_shared, int block_m,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped, PermuteSmallScratch& sc) {
  int* cnt = sc.cnt;
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < Et; e += nt) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    bool valid;
    const int e = pair_expert(ids, p, k, topk, E, &valid);
    if (valid) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  finish_offsets(cnt, sc.tcnt, sc.tmp, Et, P, block_m, expert_offsets, tiles, n_tiles, n_dropped,
                 sorted_pairs);
  // cnt now holds each expert's first sorted position: the running cursor.
  // One wavefront scatters the 64-pair groups in ascending order.
  if (tid < 64) {
    for (int p0 = 0; p0 < P; p0 += 64) {
      scatter_group(ids, p0, P, k, topk, E, cnt, sorted_pairs, pair_pos);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ---- small path, histogram form (the fused routing + permutation kernel) ---
//
// Pairs are taken in 64-pair groups, one group per wavefront at a time.  A
// pair's sorted position is the expert's first position, plus the number of
// pairs of the same expert in earlier groups (a per-group histogram, scanned
// over the groups), plus its rank among equal ids inside its own group (a
// wavefront match).  Counting uses LDS atomics, which only add, so the result
// does not depend on their order.  A handful of block barriers in total.

constexpr int kHistMaxExperts = 1032;               // E <= 1024 routed + up to 8 shared
constexpr int kHistGroups = kSmallPairs / 64;

struct PermuteHistScratch {
  int hist[kHistGroups * kHistMaxExperts];  // [group][expert]: count, then pairs in earlier groups
  int off[kHistMaxExperts + 1];             // expert -> first sorted position
  int toff[kHistMaxExperts + 1];            // expert -> first tile
  int wsum[2][16];                          // per-wavefront totals of the block scan
};

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v = dpp_add_step<0x111, 0xf>(v);   // row_shr:1
  v = dpp_add_step<0x112, 0xf>(v);   // row_shr:2
  v = dpp_add_step<0x114, 0xf>(v);   // row_shr:4
  v = dpp_add_step<0x118, 0xf>(v);   // row_shr:8   -> prefix within each row of 16
  v = dpp_add_step<0x142, 0xa>(v);   // row_bcast:15 -> rows 1, 3 add the end of rows 0, 2
  v = dpp_add_step<0x143, 0xc>(v);   // row_bcast:31 -> rows 2, 3 add the end of row 1
  return v;
}

// Exclusive prefix sums of a[0..n) and b[0..n) in LDS, in place, by the whole
// block (at most 16 wavefronts); thread i owns one contiguous run.  Returns
// both totals to every thread.  The caller synchronizes before reading.
__device__ __forceinline__ void block_scan2(int* a, int* b, int n, int (*wsum)[16], int* tot_a,
                                            int* tot_b) {
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sa = 0, sb = 0;
  for (int i = lo; i < hi; ++i) {
    sa += a[i];
    sb += b[i];
  }
  const int ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
  if (lane == 63) {
    wsum[0][w] = ia;
    wsum[1][w] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
  for (int v = 0; v < nw; ++v) {
    const int x = wsum[0][v], y = wsum[1][v];
    if (v < w) {
      pa += x;
      pb += y;
    }
    ta += x;
    tb += y;
  }
  int ra = pa + ia - sa, rb = pb + ib - sb;
  for (int i = lo; i < hi; ++i) {
    const int x = a[i], y = b[i];
    a[i] = ra;
    b[i] = rb;
    ra += x;
    rb += y;
  }
  *tot_a = ta;
  *tot_b = tb;
}

// The whole permutation of P = T * (topk + n_shared) <= kSmallPairs pairs by
// one block of a multiple of 64 threads (at most 1024); every thread calls it.
// ids may live in LDS.  Tile entries at or beyond max_tiles are not written.
__device__ __forceinline__ void permute_hist_body(
    const int32_t* ids, int T, int topk, int E, int n_shared, int block_m, int max_tiles,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped, PermuteHistScratch& sc) {
  const int k = topk + n_shared, P = T * k, Et = E + n_shared;
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63;
  const int ng = (P + 63) >> 6;
  for (int i = tid; i < ng * Et; i += nt) sc.hist[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    bool valid;
    const int e = pair_expert(ids, p, k, topk, E, &valid);
    if (valid) atomicAdd(&sc.hist[(p >> 6) * Et + e], 1);
  }
  __syncthreads();
  for (int e = tid; e < Et; e += nt) {
    int run = 0;
    for (int g = 0; g < ng; ++g) {
      const int c = sc.hist[g * Et + e];
      sc.hist[g * Et + e] = run;
      run += c;
    }
    sc.off[e] = run;
    sc.toff[e] = (run + block_m - 1) / block_m;
  }
  __syncthreads();
  int n_valid, total_tiles;
  block_scan2(sc.off, sc.toff, Et, sc.wsum, &n_valid, &total_tiles);
  __syncthreads();
  for (int pb = tid & ~63; pb < P; pb += nt) {   // whole wavefronts: the match needs every lane
    const int p = pb + lane;
    bool valid = false;
    int e = -1;
    if (p < P) e = pair_expert(ids, p, k, topk, E, &valid);
    const int key = (p >= P) ? kIdleKey : (valid ? e : kDroppedKey);
    const uint64_t peers = match_peers(key);
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (p < P) {
      if (valid) {
        const int pos = sc.off[e] + sc.hist[(p >> 6) * Et + e] + rank;
        if (pos >= 0 && pos < P) sorted_pairs[pos] = p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
    }
  }
  for (int i = max(n_valid, 0) + tid; i < P; i += nt) sorted_pairs[i] = -1;
  for (int e = tid; e < Et; e += nt) {
    const int o = sc.off[e];
    expert_offsets[e] = o;
    const int c = ((e + 1 < Et) ? sc.off[e + 1] : n_valid) - o;
    const int nte = (c + block_m - 1) / block_m;
    for (int m = 0; m < nte; ++m) {
      const int ti = sc.toff[e] + m;
      if (ti >= 0 && ti < max_tiles) {
        tiles[2 * ti] = e;
        tiles[2 * ti + 1] = m;
      }
    }
  }
  if (tid == 0) {
    expert_offsets[Et] = n_valid;
    *n_tiles = total_tiles;
    *n_dropped = P - n_valid;
  }
}

}  // namespace fp4moe
