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
#include <float.h>

#include "common.h"

namespace fp4moe {

constexpr int kRouteMaxPerLane = 16;   // E <= 1024

// float32 -> uint32 with the same order (finite inputs; +0 and -0 differ,
// but a key s + bias with s > 0 is never -0).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max(v, lane-shifted v) with DPP; lanes without a source keep v.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
  return v > t ? v : t;
}

// Maximum over the wavefront, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0x111, 0xf, 0xf>(v);   // row_shr:1
  v = dpp_max_step<0x112, 0xf, 0xf>(v);   // row_shr:2  -> lanes hold max of 4
  v = dpp_max_step<0x114, 0xf, 0xe>(v);   // row_shr:4  -> max of 8
  v = dpp_max_step<0x118, 0xf, 0xc>(v);   // row_shr:8  -> lane 15 of a row: row max
  v = dpp_max_step<0x142, 0xa, 0xf>(v);   // row_bcast:15 -> rows 1, 3 include rows 0, 2
  v = dpp_max_step<0x143, 0xc, 0xf>(v);   // row_bcast:31 -> lane 63: wavefront max
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The two largest of {a1 >= a2} and {b1 >= b2}.
__device__ __forceinline__ void merge_top2(float& a1, float& a2, float b1, float b2) {
  if (a1 >= b1) {
    a2 = fmaxf(a2, b1);
  } else {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  }
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
  const int P = (E + 63) / 64;
  const int base = lane * P;

  float sv[kRouteMaxPerLane], kv[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    sv[i] = 0.f;
    kv[i] = -FLT_MAX;
    if (i < P && base + i < E) {
      const double l = static_cast<double>(row[base + i]);
      const float s = static_cast<float>(1.0 / (1.0 + exp(-l)));   // one rounding to float32
      const float b = bias ? bias[base + i] : 0.f;
      sv[i] = s;
      kv[i] = __fadd_rn(s, b);
    }
  }

  // ---- group stage: which experts may be selected
  bool lane_kept = true;                 // aligned case: whole lane kept or not
  uint64_t kept_groups = ~0ull;          // fallback case: bit per group
  const int G = E / n_group;
  const bool aligned = n_group > 1 && (G % P) == 0 && __builtin_popcount(G / P) == 1 &&
                       (G / P) * n_group <= 64;
  if (n_group > 1 && aligned) {
    const int L = G / P;                 // lanes per group, a power of two
    float t1 = -FLT_MAX, t2 = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      if (i < P && base + i < E) {
        const float k = kv[i];
        if (k > t1) {
          t2 = t1;
          t1 = k;
        } else if (k > t2) {
          t2 = k;
        }
      }
    }
    for (int off = 1; off < L; off <<= 1) {
      const float o1 = __shfl_xor(t1, off, 64), o2 = __shfl_xor(t2, off, 64);
      merge_top2(t1, t2, o1, o2);
    }
    const float gs = __fadd_rn(t1, t2);
    const int mine = lane / L;
    int rank = 0;
    for (int g = 0; g < n_group; ++g) {
      const float o = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gs), g * L));
      rank += (o > gs || (o == gs && g < mine)) ? 1 : 0;
    }
    lane_kept = (mine < n_group) && rank < topk_group;
  } else if (n_group > 1) {
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i)
      if (i < P && base + i < E) s_key[base + i] = kv[i];
    __syncthreads();
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
    kept_groups = __ballot(keep);
  }

  // ---- selection: topk rounds of a wavefront arg-max
  uint32_t avail = 0;                    // bit i: expert base+i is a candidate
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int e = base + i;
    const bool ok = i < P && e < E && lane_kept && ((kept_groups >> (e / G)) & 1ull);
    avail |= (ok ? 1u : 0u) << i;
  }
  for (int j = 0; j < topk; ++j) {
    uint32_t best = 0;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      const uint32_t ok = order_key(kv[i]);
      if (((avail >> i) & 1u) && ok > best) {   // ascending i: strict > keeps the lower id
        best = ok;
        bi = i;
      }
    }
    const uint32_t gmax = wave_max_u32(best);
    const uint64_t win = __ballot(bi >= 0 && best == gmax);
    const int wl = __ffsll((unsigned long long)win) - 1;
    float ws = 0.f;
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < kRouteMaxPerLane; ++i)
        if (i == bi) ws = sv[i];
      avail &= ~(1u << bi);
      s_sel_idx[j] = base + bi;
      s_sel_s[j] = ws;
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
