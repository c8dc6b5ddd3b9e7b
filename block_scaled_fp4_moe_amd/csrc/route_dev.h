// Device code of moe_route: one wavefront routes one token.  Shared by the
// routing kernel and the fused small-batch routing + permutation kernel.
#pragma once
#include <float.h>

#include "common.h"

namespace fp4moe {

constexpr int kRouteMaxPerLane = 16;   // E <= 1024

// Orders this wavefront's LDS writes before its later LDS reads (the route
// scratch is private to one wavefront).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

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

// Per-wavefront LDS scratch of the routing.  Only the group stage of layouts
// whose groups are not runs of whole lanes uses it.
struct RouteScratch {
  float key[1024];
  float gscore[64];
};

// Merge with the top-2 pair held by another lane, read through DPP control CTRL.
template <int CTRL>
__device__ __forceinline__ void merge_top2_dpp(float& t1, float& t2) {
  const float o1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t1), CTRL, 0xf, 0xf, false));
  const float o2 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t2), CTRL, 0xf, 0xf, false));
  merge_top2(t1, t2, o1, o2);
}

// Routes token t with one wavefront (lane = thread index within the wave).
// Lane l owns experts [l*P, l*P + P), P = ceil(E/64) <= PM.  The selected
// ids and weights go to topk_ids / topk_w at t * topk + j and, when ids_lds
// is not NULL, the ids also to ids_lds at t * topk + j.
template <int PM>
__device__ __forceinline__ void route_token(const float* __restrict__ logits,
                                            const float* __restrict__ bias, int E, int n_group,
                                            int topk_group, int topk, int renormalize,
                                            float routed_scale, int64_t t,
                                            int32_t* __restrict__ topk_ids,
                                            float* __restrict__ topk_w, RouteScratch& sc,
                                            int* ids_lds) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + t * E;
  const int P = (E + 63) / 64;
  const int base = lane * P;

  // All loads first (clamped addresses, no branches), so that their latencies
  // overlap instead of one round trip per element.
  float lv[PM], bv[PM];
#pragma unroll
  for (int i = 0; i < PM; ++i) {
    const int e = min(base + i, E - 1);
    lv[i] = row[e];
    bv[i] = bias ? bias[e] : 0.f;
  }
  // Scores of every slot without branches (the clamped loads hold real
  // logits), so the PM exponentials are independent chains the compiler can
  // interleave; slots past E are masked afterwards.
  float sv[PM], kv[PM];
  bool have[PM];
#pragma unroll
  for (int i = 0; i < PM; ++i) {
    have[i] = i < P && base + i < E;
    const double l = static_cast<double>(lv[i]);
    const float s = static_cast<float>(1.0 / (1.0 + exp(-l)));     // one rounding to float32
    sv[i] = have[i] ? s : 0.f;
    kv[i] = have[i] ? __fadd_rn(s, bv[i]) : -FLT_MAX;
  }

  // ---- group stage: which experts may be selected
  bool lane_kept = true;                 // aligned case: whole lane kept or not
  uint64_t kept_groups = ~0ull;          // fallback case: bit per group
  const int G = E / n_group;
  const bool aligned = n_group > 1 && (G % P) == 0 && __builtin_popcount(G / P) == 1 &&
                       (G / P) * n_group <= 64 && G / P <= 32;
  if (aligned) {
    // A group is L adjacent lanes (L a power of two, at most 32); its two
    // largest keys are merged across them with DPP lane swaps.
    const int L = G / P;
    float t1 = -FLT_MAX, t2 = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < PM; ++i) {
      if (have[i]) {
        const float k = kv[i];
        if (k > t1) {
          t2 = t1;
          t1 = k;
        } else if (k > t2) {
          t2 = k;
        }
      }
    }
    if (L >= 2) merge_top2_dpp<0xB1>(t1, t2);    // quad_perm [1,0,3,2]: lane ^ 1
    if (L >= 4) merge_top2_dpp<0x4E>(t1, t2);    // quad_perm [2,3,0,1]: lane ^ 2
    if (L >= 8) merge_top2_dpp<0x141>(t1, t2);   // row_half_mirror: the other quad of 8
    if (L >= 16) merge_top2_dpp<0x140>(t1, t2);  // row_mirror: the other half of 16
    if (L >= 32) {                               // the other row of 32
      const float o1 = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t1), 0x401F));
      const float o2 = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t2), 0x401F));
      merge_top2(t1, t2, o1, o2);
    }
    const float gs = __fadd_rn(t1, t2);
    const int mine = lane / L;
    int rank = 0;
    for (int g = 0; g < n_group; ++g) {
      const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), g * L));
      rank += (o > gs || (o == gs && g < mine)) ? 1 : 0;
    }
    lane_kept = (mine < n_group) && rank < topk_group;
  } else if (n_group > 1) {
    float* s_key = sc.key;
    float* s_gscore = sc.gscore;
#pragma unroll
    for (int i = 0; i < PM; ++i)
      if (have[i]) s_key[base + i] = kv[i];
    wave_lds_sync();
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
    wave_lds_sync();
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
    wave_lds_sync();                     // the scratch may be reused by the next token
  }

  // ---- selection: topk rounds of a wavefront arg-max over order-preserving
  // integer keys (0 = not a candidate; every finite key maps above 0)
  uint32_t ok[PM];
#pragma unroll
  for (int i = 0; i < PM; ++i) {
    const int e = base + i;
    const bool cand = have[i] && lane_kept && ((kept_groups >> (min(e, E - 1) / G)) & 1ull);
    ok[i] = cand ? order_key(kv[i]) : 0u;
  }
  int my_id = 0;
  float my_s = 0.f, sum = 0.f;
  for (int j = 0; j < topk; ++j) {
    uint32_t best = ok[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < PM; ++i) {
      if (ok[i] > best) {                // ascending i: strict > keeps the lower id
        best = ok[i];
        bi = i;
      }
    }
    float s_l = sv[0];
#pragma unroll
    for (int i = 1; i < PM; ++i) s_l = (i == bi) ? sv[i] : s_l;
    const uint32_t gmax = wave_max_u32(best);
    const uint64_t win = __ballot(best == gmax);
    const int wl = __ffsll((unsigned long long)win) - 1;   // lowest lane: lowest id
    const int sel_id = __builtin_amdgcn_readlane(base + bi, wl);
    const float sel_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_l), wl));
#pragma unroll
    for (int i = 0; i < PM; ++i) ok[i] = (lane == wl && i == bi) ? 0u : ok[i];
    if (lane == j) {
      my_id = sel_id;
      my_s = sel_s;
    }
    sum = __fadd_rn(sum, sel_s);         // slot order
  }
  if (lane < topk) {
    const float w = renormalize ? __fdiv_rn(my_s, sum) : my_s;
    topk_ids[t * topk + lane] = my_id;
    topk_w[t * topk + lane] = __fmul_rn(w, routed_scale);
    if (ids_lds) ids_lds[t * topk + lane] = my_id;
  }
}

// The experts-per-lane bound a kernel is instantiated for: the smallest of
// {1, 2, 4, 6, 8, 16} that is at least ceil(E/64).
inline int route_pm(int E) {
  const int P = (E + 63) / 64;
  return P <= 1 ? 1 : P <= 2 ? 2 : P <= 4 ? 4 : P <= 6 ? 6 : P <= 8 ? 8 : 16;
}

// Expands LAUNCH(PM) for the bound route_pm(E) selects.
#define FP4MOE_ROUTE_PM_SWITCH(E, LAUNCH) \
  switch (route_pm(E)) {                  \
    case 1: LAUNCH(1); break;             \
    case 2: LAUNCH(2); break;             \
    case 4: LAUNCH(4); break;             \
    case 6: LAUNCH(6); break;             \
    case 8: LAUNCH(8); break;             \
    default: LAUNCH(16); break;           \
  }

}  // namespace fp4moe
