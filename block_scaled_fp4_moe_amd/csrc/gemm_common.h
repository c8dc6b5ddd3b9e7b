// fp4_grouped_gemm: one expert-grouped GEMM stage of the MoE layer on gfx950.
//
// [ATOM] "Stage D: MXFP4 Fused MoE": two stages, stage 1 on the fused gate/up
// weights, stage 2 on the down weights.  [ATOM] "When Is the Scale Applied?":
// for bf16 activations the block scale is absorbed while decoding the weight
// before a bf16 MFMA; for FP4 activations the payloads and E8M0 scales go
// straight into the gfx950 scaled MFMA.  [NVFP4] "Memory Management": the MoE
// path fuses dequantization into the GEMM tile, no bf16 weight buffer is
// staged in memory.  [GAUDI] "What was built": gate and up rows are
// concatenated in one fused tensor (gate first, by our reading).
//
// Operand layout of the row-major weights (the dq family and the 16x16x128
// scaled MFMA of the mx family): in a 16x16 MFMA tile lane l holds one
// 32-element MX block of row (l % 16), block index (l / 16) of the current
// 128-wide K chunk.  In the natural row-major [N, K/2] layout that is exactly
// one aligned 16-byte load per lane, with the four lanes of a row reading 64
// contiguous bytes, and its scale is one byte -- no shuffling and no LDS for
// the weights.  The accumulator of lane l holds rows 4*(l/16)..+3 (tokens) of
// column l % 16 (weight row).
//
// Families
//   dq  (wfmt MXFP4 | NVFP4 | FP8; afmt BF16, or MXFP4 with FP8 weights;
//       block_m 16 / 32, and 64 where the dqt tiles do not apply): both operands are brought to bf16 in registers
//       (v_cvt_scalef32_pk_*), then v_mfma_f32_16x16x32_bf16 with float32
//       accumulation.  The decode is exact: E2M1 x E8M0, E2M1 x E4M3 and E4M3
//       values all fit bf16.  A workgroup is four waves that split the K
//       chunks round-robin and reduce through LDS, so even a single decode
//       token spreads an expert over many CUs.  FP8 weights carry a per-row
//       float channel scale applied in the epilogue.
//   dqt (the same format pairs, and NVFP4 weights x f16 activations, with
//       block_m 64 and fragment-major weights): the dq decode in 64-row tiles
//       whose operands are staged through LDS (gemm_dqt.hip).
//   mx  (afmt MXFP4; wfmt MXFP4): v_mfma_scale_f32_*_f8f6f4 FP4 x FP4 with the
//       E8M0 bytes as the scale operands (gemm_mx.hip), up to 192 x 512 tiles.
//   f8f8 (afmt FP8; wfmt FP8; block_m 128): W8A8, the same kernel with E4M3
//       activations (one float scale per row) against E4M3 weights, both MFMA
//       format 0, 128 x 256 tiles; row and channel scales in the epilogue.
//   mx8 (afmt MXFP4; wfmt FP8; block_m 192): the 192-row scaled-MFMA tiles of
//       the mx family in the FP4 x FP8 form, E4M3 weights as MFMA format 0.
//       Only the 32x32x64 form is used: in the 16x16x128 form each FP4 lane
//       holds halves of two different 32-element K blocks, so one E8M0 scale
//       per lane could not carry an MX block.  The converted FP8 experts have
//       unit block scales and one power-of-two scale per row, which the
//       epilogue applies.  With block_m <= 64 the FP8 weights take the dq /
//       dqt decode instead.

#pragma once

#include "common.h"

namespace fp4moe {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

struct GemmParams {
  int N, K, n_experts, block_m, gather_div, w_layout, a_layout, a_rows;
  int64_t lda, ldo;
  const uint8_t* w;
  const uint8_t* w_scale;
  const float* w_tensor_scale;
  const float* w_channel_scale;
  const void* a;
  const uint8_t* a_scale;
  const int32_t* gather;
  const int32_t* offsets;
  const int32_t* tiles;
  const int32_t* n_tiles;
  uint16_t* out;
  float* out_f32;
  uint8_t* q_codes;          // stage-1 output quantized (chunk-major), or NULL
  uint8_t* q_scales;
  int q_rows;
  const float* a_f16_scale;   // FP4MOE_A_F16: the activations' power-of-two factor
  int dense_rows;             // > 0: one dense matrix of this many rows, no tile list
  const float* a_row_scale;   // FP4MOE_A_FP8: one float scale per activation row
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

__device__ __forceinline__ v8bf cat8(v2bf a, v2bf b, v2bf c, v2bf d) {
  const v4bf lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const v4bf hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E4M3FN byte -> float (finite codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// Eight bf16 weights (elements 8s..8s+7 of the lane's block) from dword `d`
// of the 16-byte E2M1 payload, times an E8M0 scale given as float.
__device__ __forceinline__ v8bf decode_mx8(uint32_t d, float scale) {
  return cat8(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3));
}

// Same for NVFP4: E2M1 times an arbitrary E4M3 scale.  The product has at
// most 6 significant bits, so it is exact in bf16.
__device__ __forceinline__ v2bf nv_pair(uint32_t d, float scale, int sel) {
  v2f f;
  switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0); break;
    case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1); break;
    case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2); break;
    default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3); break;
  }
  v2bf r;
  r[0] = (__bf16)(f[0] * scale);
  r[1] = (__bf16)(f[1] * scale);
  return r;
}

__device__ __forceinline__ v8bf decode_nv8(uint32_t d, float scale) {
  return cat8(nv_pair(d, scale, 0), nv_pair(d, scale, 1), nv_pair(d, scale, 2),
              nv_pair(d, scale, 3));
}

// NVFP4 in f16: eight E2M1 values of dword `d` (element 2i in the low nibble
// of byte i) times the E4M3 block scale given as a pair (sb, sb).  Both
// factors and the product (at most 6 significant bits: 2 of E2M1 times 4 of
// E4M3; magnitudes 2^-10 .. 2688) are exact in f16, so one conversion and one
// packed f16 multiply per pair.
__device__ __forceinline__ v8h decode_nv8_f16(uint32_t d, v2h sb2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sb2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sb2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sb2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sb2;
  const v4h lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4h hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// An E4M3 byte as the f16 pair (v, v) (exact).
__device__ __forceinline__ v2h e4m3_pair_f16(uint32_t byte) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte | (byte << 8), 1.0f, false);
}

// Eight bf16 weights from two dwords of E4M3 codes (exact).
__device__ __forceinline__ v8bf decode_fp8x8(uint32_t d0, uint32_t d1) {
  return cat8(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ v8bf as_bf8(uint4 v) { return __builtin_bit_cast(v8bf, v); }

// ---- LDS-DMA helpers (global_load_lds_*), shared by the tiled GEMMs ------

__device__ __forceinline__ uint32_t lds_offset(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

// Every lane copies 16 (4) bytes from its own global address to LDS at the
// wave-uniform byte offset `lds` + 16 (4) * lane.
// The LDS offset goes to M0 through a register constraint, so the compiler
// owns M0 (and its hazards) around the copy.
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off"
               :: "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma_b32(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off"
               :: "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maximum) as a builtin,
// so that the compiler's own wait insertion knows the LDS reads are complete.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most `newer` chunks (D DMA instructions each) issued after the
// current one are still in flight.
template <int D, int SM2>
__device__ __forceinline__ void wait_chunks(int newer) {
  if (SM2 >= 4 && newer >= 4) wait_vmcnt<(SM2 >= 4 ? 4 : 0) * D>();
  else if (SM2 >= 3 && newer == 3) wait_vmcnt<(SM2 >= 3 ? 3 : 0) * D>();
  else if (SM2 >= 2 && newer == 2) wait_vmcnt<(SM2 >= 2 ? 2 : 0) * D>();
  else if (newer == 1) wait_vmcnt<D>();
  else wait_vmcnt<0>();
}

// Workgroups that fill the device: 8 per compute unit (queried once).
int grid_cap();

// Family launchers (formats, block_m and shapes already validated).
void launch_dq_gemm(const GemmParams& p, int wfmt, int afmt, int stage, int max_tiles,
                    hipStream_t s);
void launch_mx_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s);
// Dense MXFP4 x MXFP4 (p.dense_rows rows, one fragment-major weight matrix,
// stage-2 semantics, 192 x 512 tiles).
void launch_mx_dense_gemm(const GemmParams& p, hipStream_t s);
// FP8 weights x MXFP4 activations on the scaled MFMA (block_m 192, fragment weights).
void launch_mx_fp8_wide_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s);
// FP8 weights x per-row FP8 activations (W8A8, block_m 128, fragment weights,
// chunk-major activations).
void launch_fp8_fp8_wide_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s);
// Tiled dq variant (64-row tiles, fragment weights): whether it takes `p`.
bool dqt_supported(const GemmParams& p, int stage);
void launch_dqt_gemm(const GemmParams& p, int wfmt, int afmt, int stage, int max_tiles,
                     hipStream_t s);

}  // namespace fp4moe
