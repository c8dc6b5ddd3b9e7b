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

// Routes token t with one wavefront (lane = thread index within the wave);
// the four LDS arrays are this wave's scratch: s_key[1024], s_gscore[64],
// s_sel_idx[32], s_sel_s[32].  When ids_lds is not NULL the selected ids are
// also stored there, at t * topk + j.
struct RouteScratch {
  float key[1024];
  float gscore[64];
  int sel_idx[32];
  float sel_s[32];
};

__device__ __forceinline__ void route_token(const float* __restrict__ logits,
                                            const float* __restrict__ bias, int E, int n_group,
                                            int topk_group, int topk, int renormalize,
                                            float routed_scale, int64_t t,
                                            int32_t* __restrict__ topk_ids,
                                            float* __restrict__ topk_w, RouteScratch& sc,
                                            int* ids_lds) {
  float* s_key = sc.key;
  float* s_gscore = sc.gscore;
  int* s_sel_idx = sc.sel_idx;
  float* s_sel_s = sc.sel_s;
  const int lane = threadIdx.x & 63;
  const float* row = logits + t * E;
  const int P = (E + 63) / 64;
  const int base = lane * P;

  // All loads first (clamped addresses, no branches), so that their latencies
  // overlap instead of one round trip per element.
  float lv[kRouteMaxPerLane], bv[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int e = min(base + i, E - 1);
    lv[i] = row[e];
    bv[i] = bias ? bias[e] : 0.f;
  }
  float sv[kRouteMaxPerLane], kv[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    sv[i] = 0.f;
    kv[i] = -FLT_MAX;
    if (i < P && base + i < E) {
      const double l = static_cast<double>(lv[i]);
      const float s = static_cast<float>(1.0 / (1.0 + exp(-l)));   // one rounding to float32
      sv[i] = s;
      kv[i] = __fadd_rn(s, bv[i]);
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
  wave_lds_sync();
  if (lane == 0) {
    float sum = 0.f;
    for (int j = 0; j < topk; ++j) sum = __fadd_rn(sum, s_sel_s[j]);
    for (int j = 0; j < topk; ++j) {
      const float w = renormalize ? __fdiv_rn(s_sel_s[j], sum) : s_sel_s[j];
      topk_ids[t * topk + j] = s_sel_idx[j];
      topk_w[t * topk + j] = __fmul_rn(w, routed_scale);
      if (ids_lds) ids_lds[t * topk + j] = s_sel_idx[j];
    }
  }
}

}  // namespace fp4moe
