// moe_route: grouped sigmoid top-k routing with a correction bias.
//
// [GAUDI] "What was built": grouped top-k routing, sigmoid scoring with a
// correction bias, for a DeepSeek-V3-style tower with 384 routed experts.
//
// One 64-lane wavefront routes one token.  Lane l owns the contiguous experts
// [l*P, l*P + P), P = ceil(E/64), so with E/n_group a multiple of P a group
// is a run of adjacent lanes and its score (sum of the two largest keys) is a
// short xor butterfly.  Each of the topk selection rounds is a wavefront
// maximum of an order-preserving integer image of the float32 key, computed
// with DPP row shifts and row broadcasts, then a ballot: the lowest lane
// holding the maximum owns the lowest expert id among equal keys.  Every
// decision compares float32 values, so the ids are bit-exact functions of the
// float32 scores.
#include "route_dev.h"

namespace fp4moe {

template <int PM>
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int E,
                                                   int n_group, int topk_group, int topk,
                                                   int renormalize, float routed_scale,
                                                   int32_t* __restrict__ topk_ids,
                                                   float* __restrict__ topk_w) {
  __shared__ RouteScratch scratch;
  route_token<PM>(logits, bias, E, n_group, topk_group, topk, renormalize, routed_scale, blockIdx.x,
              topk_ids, topk_w, scratch, nullptr);
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int moe_route(const float* logits, const float* bias, int T, int E, int n_group,
                         int topk_group, int topk, int renormalize, float routed_scale,
                         int32_t* topk_ids, float* topk_w, void* stream) {
  FP4MOE_REQUIRE(T >= 0, "moe_route: T=%d < 0", T);
  FP4MOE_REQUIRE(E >= 1 && E <= 64 * kRouteMaxPerLane, "moe_route: E=%d outside [1,1024]", E);
  FP4MOE_REQUIRE(n_group >= 1 && n_group <= 64 && E % n_group == 0,
                 "moe_route: n_group=%d must divide E=%d and be <= 64", n_group, E);
  FP4MOE_REQUIRE(n_group == 1 || E / n_group >= 2, "moe_route: groups need >= 2 experts");
  FP4MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, "moe_route: bad topk_group=%d",
                 topk_group);
  FP4MOE_REQUIRE(topk >= 1 && topk <= 32 && topk <= topk_group * (E / n_group),
                 "moe_route: bad topk=%d", topk);
  if (T == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(logits && topk_ids && topk_w, "moe_route: null pointer");
  FP4MOE_CHECK_DEVICE();
#define FP4MOE_ROUTE_LAUNCH(PM)                                                                 \
  hipLaunchKernelGGL(route_kernel<PM>, dim3(T), dim3(64), 0, as_stream(stream), logits, bias, E, \
                     n_group, topk_group, topk, renormalize, routed_scale, topk_ids, topk_w)
  FP4MOE_ROUTE_PM_SWITCH(E, FP4MOE_ROUTE_LAUNCH)
#undef FP4MOE_ROUTE_LAUNCH
  return check_launch("moe_route");
}
