// moe_route: grouped sigmoid top-k routing with a correction bias.
//
// [GAUDI] "What was built": grouped top-k routing, sigmoid scoring with a
// correction bias, for a DeepSeek-V3-style tower with 384 routed experts.
// One 64-lane wavefront routes one token.  Lane l owns experts l, l+64, ...;
// every selection decision compares float32 keys with index tie-breaks, so
// the ids are bit-exact functions of the float32 scores.
#include <float.h>
#include <limits.h>

#include "common.h"

namespace fp4moe {

constexpr int kRouteMaxPerLane = 16;   // E <= 1024

struct Cand {
  float key;
  float s;
  int idx;
};

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int E,
                                                   int n_group, int topk_group, int topk,
                                                   int renormalize, float routed_scale,
                                                   int32_t* __restrict__ topk_ids,
                                                   float* __restrict__ topk_w) {
  __shared__ float s_key[1024];
  __shared__ float s_gscore[64];
  __shared__ int s_sel_idx[32];
  __shared__ float s_sel_s[32];

  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const float* row = logits + t * E;

  float sv[kRouteMaxPerLane], kv[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    sv[i] = 0.f;
    kv[i] = -FLT_MAX;
    if (e < E) {
      const double l = static_cast<double>(row[e]);
      const float s = static_cast<float>(1.0 / (1.0 + exp(-l)));   // one rounding to float32
      const float b = bias ? bias[e] : 0.f;
      const float key = __fadd_rn(s, b);
      sv[i] = s;
      kv[i] = key;
      s_key[e] = key;
    }
  }
  __syncthreads();

  // Group stage: lane g scores group g by the sum of its two largest keys.
  uint64_t kept = ~0ull;
  int G = E;
  if (n_group > 1) {
    G = E / n_group;
    float gs = -FLT_MAX;
    if (lane < n_group) {
      float t1 = -FLT_MAX, t2 = -FLT_MAX;
      for (int j = 0; j < G; ++j) {
        const float k = s_key[lane * G + j];
        if (k > t1) {
          t2 = t1;
          t1 = k;
        } else if (k > t2) {
          t2 = k;
        }
      }
      gs = __fadd_rn(t1, t2);
      s_gscore[lane] = gs;
    }
    __syncthreads();
    bool keep = false;
    if (lane < n_group) {
      int rank = 0;
      for (int g = 0; g < n_group; ++g) {
        const float o = s_gscore[g];
        rank += (o > gs || (o == gs && g < lane)) ? 1 : 0;
      }
      keep = rank < topk_group;
    }
    kept = __ballot(keep);
  }

  // Expert stage: topk rounds of a wavefront arg-max over the allowed experts.
  uint32_t taken = 0;
  for (int j = 0; j < topk; ++j) {
    float bk = -FLT_MAX, bs = 0.f;
    int bi = INT_MAX;
    bool have = false;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && ((kept >> (e / G)) & 1ull)) {
        if (!have || kv[i] > bk) {   // ascending e: strict > keeps the lower id on ties
          bk = kv[i];
          bs = sv[i];
          bi = e;
          have = true;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off, 64);
      const float os = __shfl_xor(bs, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bs = os;
        bi = oi;
      }
    }
    if (bi != INT_MAX && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      s_sel_idx[j] = bi;
      s_sel_s[j] = bs;
    }
  }
  __syncthreads();
  if (lane == 0) {
    float sum = 0.f;
    for (int j = 0; j < topk; ++j) sum = __fadd_rn(sum, s_sel_s[j]);
    for (int j = 0; j < topk; ++j) {
      const float w = renormalize ? __fdiv_rn(s_sel_s[j], sum) : s_sel_s[j];
      topk_ids[t * topk + j] = s_sel_idx[j];
      topk_w[t * topk + j] = __fmul_rn(w, routed_scale);
    }
  }
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
  hipLaunchKernelGGL(route_kernel, dim3(T), dim3(64), 0, as_stream(stream), logits, bias, E,
                     n_group, topk_group, topk, renormalize, routed_scale, topk_ids, topk_w);
  return check_launch("moe_route");
}
