// moe_decode_fused: the whole decode MoE layer (bf16 activations, MXFP4
// weights) in one launch, for batches of at most 16 tokens.
//
// [GAUDI] "What was built": decode kernels for at most 16 tokens that touch
// only the routed experts.  [ATOM] "Stage D: MXFP4 Fused MoE": the small-token
// moe2 variant reduces the experts' outputs into the token rows inside the
// down GEMM instead of a separate combine pass.  [K3] "Copy inputs only for
// kernels that use them": at small batch sizes fixed per-launch costs dominate.
//
// One cooperative launch (every workgroup resident at once, so the grid
// barrier below cannot wait on a workgroup that was never scheduled):
//   1. every workgroup routes the T tokens itself (the moe_route device code,
//      one wavefront per token) and sorts the T*k pairs by expert in LDS
//      (stable, block_m 16); workgroup 0 also writes both results out;
//   2. stage 1: the dq work items (one 16-row expert tile x 32 output columns)
//      of gate/up + SiLU*up, the workgroups looping over them; h to memory;
//   3. a grid barrier (an arrival counter and a generation word in the
//      caller's workspace; a bounded wait that raises a flag instead of
//      hanging);
//   4. stage 2: the dq work items (one tile x 64 output columns); y to memory.
//      The item that completes a column block last (a per-block counter in the
//      workspace) adds the block's y rows into every token's output in slot
//      order, exactly as moe_combine does, and resets the counter.
// No step depends on the order in which workgroups arrive, so the result is
// bit-identical to moe_route_permute + fp4_grouped_gemm (dq, block_m 16) x 2 +
// moe_combine on the same inputs.
#include <mutex>

#include "dq_item.h"
#include "permute_dev.h"
#include "route_dev.h"

namespace fp4moe {

constexpr int kFusedTokens = 16;
constexpr int kFusedTopk = 16;
constexpr int kFusedPairs = kFusedTokens * (kFusedTopk + 8);
constexpr int kFusedWaves = 4;
constexpr int kFusedBM = 16;
// workspace words: [0] arrivals, [1] generation, [2] timeout flag, [3] unused,
// [4 + b] finished stage-2 items of output column block b
constexpr int kSyncHeader = 4;
// bounded barrier wait: about a second of s_sleep before the flag is raised
constexpr uint32_t kSpinLimit = 1u << 23;

struct FusedLds {
  union {
    RouteScratch route[kFusedWaves];
    float red[kFusedWaves - 1][4 * 4][64];   // dq reduction (one M block, four groups)
  } u;
  int32_t ids[kFusedTokens * kFusedTopk];
  float wts[kFusedTokens * kFusedTopk];
  int32_t off[kHistMaxExperts + 1];   // counts, then first sorted row per expert
  int32_t toff[kHistMaxExperts + 1];  // tiles per expert, then first tile
  int32_t spair[kFusedPairs];
  int32_t ppos[kFusedPairs];
  int32_t tiles[2 * kFusedPairs];
  int32_t wsum[2][16];
  int32_t ntiles, nvalid, last;
};

struct DecodeParams {
  int T, H, I, E, n_shared, n_group, topk_group, topk, renormalize, max_tiles;
  float routed_scale;
  const uint16_t* x;
  const float* logits;
  const float* bias;
  const uint8_t* w13;
  const uint8_t* w13_scale;
  const uint8_t* w2;
  const uint8_t* w2_scale;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* sorted_pairs;
  int32_t* pair_pos;
  int32_t* tiles;
  int32_t* n_tiles;
  int32_t* n_dropped;
  uint16_t* h;
  uint16_t* y;
  uint16_t* out;
  uint32_t* sync;
};

// Every workgroup of the grid waits here until all have arrived.  Stores made
// before the barrier are visible to loads made after it (agent-scope fences
// around the counter).
__device__ __forceinline__ void grid_barrier(uint32_t* sync) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t gen = __hip_atomic_load(&sync[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t n =
        __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (n == gridDim.x - 1) {
      __hip_atomic_store(&sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&sync[1], gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // relaxed loads while waiting: an acquire on every iteration would
      // invalidate this XCD's L2 under the workgroups still streaming weights
      uint32_t spins = 0;
      while (__hip_atomic_load(&sync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(4);
        if (++spins == kSpinLimit) {
          __hip_atomic_store(&sync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // every workgroup's stores before it
  }
  __syncthreads();
}

template <int PM>
__global__ __launch_bounds__(64 * kFusedWaves, 4) void decode_fused_kernel(DecodeParams a) {
  __shared__ FusedLds L;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int topk = a.topk, k = topk + a.n_shared, P = a.T * k, Et = a.E + a.n_shared;

  // ---- 1. routing of every token, then the stable sort of the pairs
  for (int t = wave; t < a.T; t += kFusedWaves)
    route_token<PM>(a.logits, a.bias, a.E, a.n_group, a.topk_group, topk, a.renormalize,
                    a.routed_scale, t, L.ids, L.wts, L.u.route[wave], nullptr);
  for (int e = tid; e < Et; e += blockDim.x) L.off[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    bool valid;
    const int e = pair_expert(L.ids, p, k, topk, a.E, &valid);
    if (valid) atomicAdd(&L.off[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < Et; e += blockDim.x) L.toff[e] = (L.off[e] + kFusedBM - 1) / kFusedBM;
  __syncthreads();
  int nvalid, ntiles;
  block_scan2(L.off, L.toff, Et, L.wsum, &nvalid, &ntiles);
  __syncthreads();
  if (tid == 0) {
    L.off[Et] = nvalid;
    L.ntiles = ntiles;
  }
  // sorted position of pair p: its expert's first row plus the pairs of the
  // same expert before it (pairs are few, so a direct count)
  for (int p = tid; p < P; p += blockDim.x) {
    bool valid;
    const int e = pair_expert(L.ids, p, k, topk, a.E, &valid);
    if (!valid) {
      L.ppos[p] = -1;
      continue;
    }
    int rank = 0;
    for (int q = 0; q < p; ++q) {
      bool vq;
      rank += (pair_expert(L.ids, q, k, topk, a.E, &vq) == e && vq) ? 1 : 0;
    }
    const int pos = L.off[e] + rank;
    L.ppos[p] = pos;
    L.spair[pos] = p;
  }
  for (int i = nvalid + tid; i < P; i += blockDim.x) L.spair[i] = -1;
  __syncthreads();
  for (int e = tid; e < Et; e += blockDim.x) {
    const int c = L.off[e + 1] - L.off[e];
    for (int m = 0; m * kFusedBM < c; ++m) {
      L.tiles[2 * (L.toff[e] + m)] = e;
      L.tiles[2 * (L.toff[e] + m) + 1] = m;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.T * topk; i += blockDim.x) {
      a.topk_ids[i] = L.ids[i];
      a.topk_w[i] = L.wts[i];
    }
    for (int e = tid; e <= Et; e += blockDim.x) a.expert_offsets[e] = L.off[e];
    for (int p = tid; p < P; p += blockDim.x) {
      a.sorted_pairs[p] = L.spair[p];
      a.pair_pos[p] = L.ppos[p];
    }
    for (int i = tid; i < ntiles && i < a.max_tiles; i += blockDim.x) {
      a.tiles[2 * i] = L.tiles[2 * i];
      a.tiles[2 * i + 1] = L.tiles[2 * i + 1];
    }
    if (tid == 0) {
      *a.n_tiles = ntiles;
      *a.n_dropped = P - nvalid;
    }
  }

  // ---- 2. stage 1 (the permutation above lives in LDS; dq_item reads it there)
  GemmParams p{};
  p.N = 2 * a.I;
  p.K = a.H;
  p.n_experts = Et;
  p.block_m = kFusedBM;
  p.gather_div = k;
  p.w_layout = FP4MOE_LAYOUT_FRAGMENT;
  p.a_layout = FP4MOE_A_LAYOUT_ROWMAJOR;
  p.lda = a.H;
  p.ldo = a.I;
  p.w = a.w13;
  p.w_scale = a.w13_scale;
  p.a = a.x;
  p.gather = L.spair;
  p.offsets = L.off;
  p.tiles = L.tiles;
  p.n_tiles = &L.ntiles;
  p.out = a.h;
  const int64_t n1 = (int64_t)ntiles * (a.I / dq_out_cols<1, 4>());
  for (int64_t wi = blockIdx.x; wi < n1; wi += gridDim.x)
    dq_item<FP4MOE_W_MXFP4, FP4MOE_A_BF16, 1, 1, 4, 2, kFusedWaves>(p, wi, L.u.red);

  // ---- 3. every row of h is written before any stage-2 item reads it
  grid_barrier(a.sync);

  // ---- 4. stage 2 and the combine
  p.N = a.H;
  p.K = a.I;
  p.gather = nullptr;
  p.gather_div = 1;
  p.lda = a.I;
  p.ldo = a.H;
  p.w = a.w2;
  p.w_scale = a.w2_scale;
  p.a = a.h;
  p.out = a.y;
  constexpr int COLS = dq_out_cols<2, 4>();
  const int n_nb = a.H / COLS;
  uint32_t* done = a.sync + kSyncHeader;
  const int64_t n2 = (int64_t)ntiles * n_nb;
  for (int64_t wi = blockIdx.x; wi < n2; wi += gridDim.x) {
    dq_item<FP4MOE_W_MXFP4, FP4MOE_A_BF16, 2, 1, 4, 2, kFusedWaves>(p, wi, L.u.red);
    const int nb = (int)(wi % n_nb);
    if (tid == 0) {
      // release: this item's y rows (stored by this wave) before the count
      const uint32_t d =
          __hip_atomic_fetch_add(&done[nb], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      L.last = (d == (uint32_t)ntiles - 1u);
    }
    __syncthreads();
    if (L.last) {
      // acquire: every other item's y rows of this block
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // out[t] = bf16(sum_j w[t,j] * y[pos(t,j)]) over ascending slots, 8 columns per thread
      for (int idx = tid; idx < a.T * (COLS / 8); idx += blockDim.x) {
        const int t = idx / (COLS / 8);
        const int col = nb * COLS + (idx % (COLS / 8)) * 8;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j < k; ++j) {
          const int pp = L.ppos[t * k + j];
          if (pp < 0) continue;
          const float w = (j < topk) ? L.wts[t * topk + j] : 1.f;
          const uint4 v = *reinterpret_cast<const uint4*>(a.y + (int64_t)pp * a.H + col);
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, bf16_to_f32(u[i] & 0xffffu), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
          }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.H + col) =
            make_uint4(o[0], o[1], o[2], o[3]);
      }
      if (tid == 0) __hip_atomic_store(&done[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
}

// Co-resident workgroups of one instantiation on the current device (cached).
template <int PM>
static int fused_grid(int dev) {
  static std::mutex mu;
  static int cache[64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_fused_kernel<PM>,
                                                     64 * kFusedWaves, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <int PM>
static int launch_fused(const DecodeParams& a, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_error(FP4MOE_ERR_UNSUPPORTED, "no device");
  const int grid = fused_grid<PM>(dev);
  if (grid <= 0)
    return set_error(FP4MOE_ERR_LAUNCH, "moe_decode_fused: occupancy query failed");
  DecodeParams arg = a;
  void* args[] = {&arg};
  const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(
                                                      decode_fused_kernel<PM>),
                                                  dim3(grid), dim3(64 * kFusedWaves), args, 0, s);
  if (e != hipSuccess)
    return set_error(FP4MOE_ERR_LAUNCH, "moe_decode_fused: %s", hipGetErrorString(e));
  return check_launch("moe_decode_fused");
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" size_t moe_decode_fused_workspace(int H) {
  if (H <= 0) return 0;
  return (size_t)(kSyncHeader + (H + 63) / 64) * sizeof(uint32_t);
}

extern "C" int moe_decode_fused(const fp4moe_decode_args* a, void* stream) {
  FP4MOE_REQUIRE(a, "moe_decode_fused: null args");
  FP4MOE_REQUIRE(a->T >= 0 && a->T <= kFusedTokens, "moe_decode_fused: T=%d outside [0,%d]",
                 a->T, kFusedTokens);
  FP4MOE_REQUIRE(a->E >= 1 && a->E <= 64 * kRouteMaxPerLane,
                 "moe_decode_fused: E=%d outside [1,1024]", a->E);
  FP4MOE_REQUIRE(a->n_group >= 1 && a->n_group <= 64 && a->E % a->n_group == 0 &&
                     (a->n_group == 1 || a->E / a->n_group >= 2),
                 "moe_decode_fused: n_group=%d for E=%d", a->n_group, a->E);
  FP4MOE_REQUIRE(a->topk_group >= 1 && a->topk_group <= a->n_group,
                 "moe_decode_fused: topk_group=%d", a->topk_group);
  FP4MOE_REQUIRE(a->topk >= 1 && a->topk <= kFusedTopk &&
                     a->topk <= a->topk_group * (a->E / a->n_group),
                 "moe_decode_fused: topk=%d", a->topk);
  FP4MOE_REQUIRE(a->n_shared >= 0 && a->n_shared <= 8, "moe_decode_fused: n_shared=%d",
                 a->n_shared);
  FP4MOE_REQUIRE(a->E + a->n_shared <= kHistMaxExperts, "moe_decode_fused: E+n_shared=%d above %d",
                 a->E + a->n_shared, kHistMaxExperts);
  FP4MOE_REQUIRE(a->H > 0 && a->H % 128 == 0 && a->I > 0 && a->I % 128 == 0,
                 "moe_decode_fused: H=%d and I=%d must be multiples of 128", a->H, a->I);
  const int max_tiles = moe_permute_max_tiles(a->T, a->topk, a->E, a->n_shared, kFusedBM);
  FP4MOE_REQUIRE(a->max_tiles >= max_tiles, "moe_decode_fused: max_tiles=%d < %d",
                 a->max_tiles, max_tiles);
  if (a->workspace_bytes < moe_decode_fused_workspace(a->H))
    return set_error(FP4MOE_ERR_WORKSPACE, "moe_decode_fused: workspace %zu < %zu bytes",
                     a->workspace_bytes, moe_decode_fused_workspace(a->H));
  if (a->T == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(a->x && a->logits && a->w13 && a->w13_scale && a->w2 && a->w2_scale &&
                     a->topk_ids && a->topk_w && a->expert_offsets && a->sorted_pairs &&
                     a->pair_pos && a->tiles && a->n_tiles && a->n_dropped && a->h && a->y &&
                     a->out && a->workspace,
                 "moe_decode_fused: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)a->x & 15) == 0 && ((uintptr_t)a->w13 & 15) == 0 &&
                     ((uintptr_t)a->w2 & 15) == 0 && ((uintptr_t)a->h & 15) == 0 &&
                     ((uintptr_t)a->y & 15) == 0 && ((uintptr_t)a->out & 15) == 0 &&
                     ((uintptr_t)a->workspace & 3) == 0,
                 "moe_decode_fused: x, weights, h, y and out must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  DecodeParams d{};
  d.T = a->T;
  d.H = a->H;
  d.I = a->I;
  d.E = a->E;
  d.n_shared = a->n_shared;
  d.n_group = a->n_group;
  d.topk_group = a->topk_group;
  d.topk = a->topk;
  d.renormalize = a->renormalize;
  d.max_tiles = a->max_tiles;
  d.routed_scale = a->routed_scale;
  d.x = a->x;
  d.logits = a->logits;
  d.bias = a->bias;
  d.w13 = a->w13;
  d.w13_scale = a->w13_scale;
  d.w2 = a->w2;
  d.w2_scale = a->w2_scale;
  d.topk_ids = a->topk_ids;
  d.topk_w = a->topk_w;
  d.expert_offsets = a->expert_offsets;
  d.sorted_pairs = a->sorted_pairs;
  d.pair_pos = a->pair_pos;
  d.tiles = a->tiles;
  d.n_tiles = a->n_tiles;
  d.n_dropped = a->n_dropped;
  d.h = a->h;
  d.y = a->y;
  d.out = a->out;
  d.sync = static_cast<uint32_t*>(a->workspace);
  hipStream_t s = as_stream(stream);
#define FP4MOE_FUSED_LAUNCH(PM) return launch_fused<PM>(d, s)
  FP4MOE_ROUTE_PM_SWITCH(a->E, FP4MOE_FUSED_LAUNCH)
#undef FP4MOE_FUSED_LAUNCH
  return FP4MOE_OK;
}
