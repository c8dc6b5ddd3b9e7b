// moe_route_permute: moe_route followed by moe_permute in one launch, for
// batches of at most 1024 (token, slot) pairs (the decode sizes).
//
// One workgroup of up to 16 wavefronts.  Each wavefront routes tokens (the
// same device code as moe_route), the selected ids stay in LDS, and the
// workgroup then sorts the pairs by expert with per-group histograms and
// wavefront matches (a few block barriers in all).  At decode sizes both steps
// are latency bound: one launch instead of two removes a kernel start and the
// dependency gap between the kernels.
#include <algorithm>

#include "permute_dev.h"
#include "route_dev.h"

namespace fp4moe {

constexpr int kFusedMaxWaves = 16;

// Wavefronts per workgroup: 16, or 8 for the widest routing layout (E > 512),
// whose registers would not fit 16.
constexpr int fused_max_waves(int pm) { return pm >= 16 ? 8 : kFusedMaxWaves; }

template <int PM>
__global__ __launch_bounds__(64 * fused_max_waves(PM)) void route_permute_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int n_group,
    int topk_group, int topk, int renormalize, float routed_scale, int n_shared, int block_m,
    int max_tiles, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ n_dropped) {
  // The routing scratch is dead once every token is routed, so the
  // permutation's scratch reuses it.
  __shared__ union {
    RouteScratch route[kFusedMaxWaves];
    PermuteHistScratch perm;
  } scratch;
  __shared__ int ids_lds[kSmallPairs];
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int t = wave; t < T; t += nw)
    route_token<PM>(logits, bias, E, n_group, topk_group, topk, renormalize, routed_scale, t,
                    topk_ids, topk_w, scratch.route[wave], ids_lds);
  __syncthreads();
  permute_hist_body(ids_lds, T, topk, E, n_shared, block_m, max_tiles, expert_offsets,
                    sorted_pairs, pair_pos, tiles, n_tiles, n_dropped, scratch.perm);
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int moe_route_permute(const float* logits, const float* bias, int T, int E,
                                 int n_group, int topk_group, int topk, int renormalize,
                                 float routed_scale, int n_shared, int block_m,
                                 int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                 int32_t* sorted_pairs, int32_t* pair_pos, int32_t* tiles,
                                 int32_t* n_tiles, int32_t* n_dropped, void* stream) {
  FP4MOE_REQUIRE(T >= 0, "moe_route_permute: T=%d < 0", T);
  FP4MOE_REQUIRE(E >= 1 && E <= 64 * kRouteMaxPerLane, "moe_route_permute: E=%d outside [1,1024]",
                 E);
  FP4MOE_REQUIRE(n_group >= 1 && n_group <= 64 && E % n_group == 0,
                 "moe_route_permute: n_group=%d must divide E=%d and be <= 64", n_group, E);
  FP4MOE_REQUIRE(n_group == 1 || E / n_group >= 2, "moe_route_permute: groups need >= 2 experts");
  FP4MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, "moe_route_permute: bad topk_group=%d",
                 topk_group);
  FP4MOE_REQUIRE(topk >= 1 && topk <= 32 && topk <= topk_group * (E / n_group),
                 "moe_route_permute: bad topk=%d", topk);
  FP4MOE_REQUIRE(n_shared >= 0 && n_shared <= 8, "moe_route_permute: n_shared=%d outside [0,8]",
                 n_shared);
  FP4MOE_REQUIRE(E + n_shared <= kHistMaxExperts, "moe_route_permute: E+n_shared=%d above %d",
                 E + n_shared, kHistMaxExperts);
  FP4MOE_REQUIRE(block_m >= 1 && block_m <= 1024, "moe_route_permute: block_m=%d", block_m);
  FP4MOE_REQUIRE((int64_t)T * (topk + n_shared) <= kSmallPairs,
                 "moe_route_permute: T*(topk+n_shared)=%lld above %d (use moe_route and "
                 "moe_permute)", (long long)T * (topk + n_shared), kSmallPairs);
  FP4MOE_REQUIRE(expert_offsets && n_tiles && n_dropped, "moe_route_permute: null output pointer");
  FP4MOE_REQUIRE(T == 0 || (logits && topk_ids && topk_w && sorted_pairs && pair_pos && tiles),
                 "moe_route_permute: null pointer");
  FP4MOE_CHECK_DEVICE();
  // One wavefront per token while they last, at least one per 64 pairs, and at
  // least 8 so the per-expert loops of the permutation stay short; up to the
  // workgroup's limit (the loops stride over the rest).
  const int P = T * (topk + n_shared);
  const int nw = std::min(fused_max_waves(route_pm(E)), std::max({8, T, (P + 63) / 64}));
  const int max_tiles = moe_permute_max_tiles(T, topk, E, n_shared, block_m);
#define FP4MOE_RP_LAUNCH(PM)                                                                    \
  hipLaunchKernelGGL(route_permute_kernel<PM>, dim3(1), dim3(64 * nw), 0, as_stream(stream),    \
                     logits, bias, T, E, n_group, topk_group, topk, renormalize, routed_scale,  \
                     n_shared, block_m, max_tiles, topk_ids, topk_w, expert_offsets,            \
                     sorted_pairs, pair_pos, tiles, n_tiles, n_dropped)
  FP4MOE_ROUTE_PM_SWITCH(E, FP4MOE_RP_LAUNCH)
#undef FP4MOE_RP_LAUNCH
  return check_launch("moe_route_permute");
}
