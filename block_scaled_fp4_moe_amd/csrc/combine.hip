// moe_combine: weighted top-k combine of the stage-2 rows.
//
// [ATOM] "Stage D: MXFP4 Fused MoE": the stage-2 outputs of a token's expert
// pairs are reduced into the token's output row.  [K3]: the shared-expert
// contribution is added to the routed sum.
// out[t] = bf16( sum_{j<topk} w[t,j] * y[pos(t,j)] + sum_i y[pos(t,topk+i)] ),
// accumulated in float32 in ascending slot order (deterministic, no atomics).
// Each lane owns 8 consecutive columns (16-byte loads and stores).
#include "common.h"

namespace fp4moe {

// Each stage-2 row is read once here: the streaming (non-temporal) form of
// the 16-byte load measured 13% faster on the T=8192 layer than cached loads.
__device__ __forceinline__ uint4 load_once16(const uint16_t* ptr) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr)));
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int topk,
                                                      int n_shared, int H,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32, int T) {
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (col >= H) return;
  const int k = topk + n_shared;
  // grid y covers at most 65535 tokens; each y index strides over the rest
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // Slots in batches of 8: all row loads of a batch are issued before the
  // batch is accumulated, in ascending slot order.
  for (int j0 = 0; j0 < k; j0 += 8) {
    uint4 v[8];
    float w[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      const int p = (j < k) ? pair_pos[t * k + j] : -1;
      w[jj] = (p < 0) ? 0.f : ((j < topk) ? topk_w[t * topk + j] : 1.f);
      v[jj] = (p < 0) ? make_uint4(0, 0, 0, 0)
                      : load_once16(y + (int64_t)p * H + col);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj >= k) break;
      const uint32_t u[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w[jj], bf16_to_f32(u[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w[jj], bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(out + t * H + col) = make_uint4(o[0], o[1], o[2], o[3]);
  if (out_f32) {
    float4* of = reinterpret_cast<float4*>(out_f32 + t * H + col);
    of[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    of[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  }
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int moe_combine(const uint16_t* y_sorted, const int32_t* pair_pos, const float* topk_w,
                           int T, int topk, int n_shared, int H, uint16_t* out, float* out_f32,
                           void* stream) {
  FP4MOE_REQUIRE(T >= 0 && topk >= 1 && n_shared >= 0 && H > 0 && H % 8 == 0,
                 "moe_combine: T=%d topk=%d n_shared=%d H=%d (H %% 8 != 0)", T, topk, n_shared, H);
  if (T == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(y_sorted && pair_pos && topk_w && out, "moe_combine: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)y_sorted & 15) == 0 && ((uintptr_t)out & 15) == 0 &&
                     ((uintptr_t)out_f32 & 15) == 0,
                 "moe_combine: y, out and out_f32 must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  const int lanes = H / 8;
  dim3 grid((lanes + 255) / 256, T < 65535 ? T : 65535);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, as_stream(stream), y_sorted, pair_pos,
                     topk_w, topk, n_shared, H, out, out_f32, T);
  return check_launch("moe_combine");
}
