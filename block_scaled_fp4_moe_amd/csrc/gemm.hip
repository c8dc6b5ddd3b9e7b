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
// Operand layout (both MFMA families): in a 16x16 MFMA tile lane l holds one
// 32-element MX block of row (l % 16), block index (l / 16) of the current
// 128-wide K chunk.  In the natural row-major [N, K/2] layout that is exactly
// one aligned 16-byte load per lane, with the four lanes of a row reading 64
// contiguous bytes, and its scale is one byte -- no shuffling and no LDS for
// the weights.  The accumulator of lane l holds rows 4*(l/16)..+3 (tokens) of
// column l % 16 (weight row).
//
// Families
//   dq  (wfmt MXFP4 | NVFP4 | FP8; afmt BF16, or MXFP4 with FP8 weights):
//       both operands are brought to bf16 in registers (v_cvt_scalef32_pk_*),
//       then v_mfma_f32_16x16x32_bf16 with float32 accumulation.  The decode is
//       exact: E2M1 x E8M0, E2M1 x E4M3 and E4M3 values all fit bf16.  A
//       workgroup is four waves that split the K chunks round-robin and reduce
//       through LDS, so even a single decode token spreads an expert over many
//       CUs.  FP8 weights carry a per-row float channel scale applied in the
//       epilogue.
//   mx  (afmt MXFP4; wfmt MXFP4): v_mfma_scale_f32_16x16x128_f8f6f4 FP4 x FP4
//       with the E8M0 bytes as the scale operands.
//
// FP8 weights with MXFP4 activations go through the bf16 path on purpose: in
// the mixed FP4 x FP8 form of the scaled MFMA each FP4 lane holds halves of
// two different 32-element K blocks, so one E8M0 scale per lane cannot carry
// an MX block scale there.  The bf16 path computes the same exact products.
#include "common.h"

namespace fp4moe {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct GemmParams {
  int N, K, n_experts, block_m, gather_div, w_layout;
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

// ===========================================================================
// dq family: bf16 activations, FP4 weights decoded in registers
// ===========================================================================

template <int WFMT, int AFMT, int STAGE, int MB>
__global__ __launch_bounds__(256) void dq_gemm_kernel(GemmParams p) {
  constexpr int NG = 2;            // two 16-row weight groups per work item
  constexpr int U = (MB == 1) ? 4 : (MB == 2 ? 2 : 1);   // chunks in flight per wave
  constexpr int NV = MB * NG * 4;  // accumulator floats per lane
  __shared__ float red[3][NV][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int BM = MB * 16;
  const int n_nb = (STAGE == 1) ? (p.N / 2) / 16 : p.N / 32;
  const int nkc = p.K / 128;
  const int64_t wrow_bytes = (WFMT == FP4MOE_W_FP8) ? p.K : p.K / 2;
  const int64_t srow_bytes = (WFMT == FP4MOE_W_MXFP4) ? p.K / 32 : p.K / 16;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;

  for (int64_t wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
    const int tile = (int)(wi / n_nb), nb = (int)(wi - (int64_t)tile * n_nb);
    const int e = p.tiles[2 * tile], mt = p.tiles[2 * tile + 1];
    const int row0 = p.offsets[e] + mt * BM;
    const int row_end = min(p.offsets[e + 1], row0 + BM);

    // Per lane and weight group: code / scale address of chunk 0 and the
    // stride between chunks, for the row-major or the fragment-major layout.
    const uint8_t* wp[NG];
    const uint8_t* sp[NG];
    int wrow[NG];
    int64_t wstride, sstride, whalf;
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
      const int wr = (STAGE == 1) ? (ng * (p.N / 2) + nb * 16 + r16) : (nb * 32 + ng * 16 + r16);
      wrow[ng] = wr;
      if (p.w_layout == 0) {
        const int64_t row = (int64_t)e * p.N + wr;
        wp[ng] = p.w + row * wrow_bytes + g * (WFMT == FP4MOE_W_FP8 ? 32 : 16);
        sp[ng] = (WFMT == FP4MOE_W_FP8) ? nullptr
                                        : p.w_scale + row * srow_bytes + g * (WFMT == FP4MOE_W_MXFP4 ? 1 : 2);
        wstride = (WFMT == FP4MOE_W_FP8) ? 128 : 64;
        whalf = 16;
        sstride = (WFMT == FP4MOE_W_MXFP4) ? 4 : 8;
      } else {
        const int64_t f0 = ((int64_t)e * (p.N / 16) + wr / 16) * nkc;
        wstride = (WFMT == FP4MOE_W_FP8) ? 2048 : 1024;
        whalf = 1024;
        wp[ng] = p.w + f0 * wstride + lane * 16;
        // scales are chunk-major: (e*C + c)*G + group
        const int sfrag = (WFMT == FP4MOE_W_MXFP4) ? 64 : 128;
        sstride = (int64_t)(p.N / 16) * sfrag;
        sp[ng] = (WFMT == FP4MOE_W_FP8)
                     ? nullptr
                     : p.w_scale + ((int64_t)e * nkc * (p.N / 16) + wr / 16) * sfrag +
                           lane * (WFMT == FP4MOE_W_MXFP4 ? 1 : 2);
      }
    }
    // A rows: bf16 [., lda] or MXFP4 codes [., lda/2] + E8M0 [., lda/32]
    const uint8_t* ap[MB];
    const uint8_t* asp[MB];
    bool av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = row0 + mb * 16 + r16;
      av[mb] = r < row_end;
      int64_t arow = r;
      if (av[mb] && p.gather) arow = p.gather[r] / p.gather_div;
      if (!av[mb]) arow = 0;
      if (AFMT == FP4MOE_A_BF16) {
        ap[mb] = static_cast<const uint8_t*>(p.a) + arow * p.lda * 2;
        asp[mb] = nullptr;
      } else {
        ap[mb] = static_cast<const uint8_t*>(p.a) + arow * (p.lda / 2);
        asp[mb] = p.a_scale + arow * (p.lda / 32);
      }
    }

    v4f acc[MB][NG];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) acc[mb][ng] = v4f{0.f, 0.f, 0.f, 0.f};

    // K chunks go round-robin over the four waves; each step of a wave takes
    // U of its chunks and issues all their loads before the first MFMA, so a
    // wave keeps U*NG 16-byte weight loads per lane in flight.
    for (int c0 = wave; c0 < nkc; c0 += 4 * U) {
      uint4 wv[U][NG][2];
      float sc[U][NG][2];
      uint4 a4[U][MB][4];
      float asc[U][MB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 4 * u;
        if (c >= nkc) break;
        const int blk = c * 4 + g;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          const uint8_t* wc = wp[ng] + (int64_t)c * wstride;
          if (WFMT == FP4MOE_W_FP8) {
            wv[u][ng][0] = *reinterpret_cast<const uint4*>(wc);
            wv[u][ng][1] = *reinterpret_cast<const uint4*>(wc + whalf);
            sc[u][ng][0] = sc[u][ng][1] = 1.0f;
          } else {
            wv[u][ng][0] = *reinterpret_cast<const uint4*>(wc);
            wv[u][ng][1] = wv[u][ng][0];
            const uint8_t* scp = sp[ng] + (int64_t)c * sstride;
            if (WFMT == FP4MOE_W_MXFP4) {
              // the convert takes the float's exponent field as an E8M0 byte
              sc[u][ng][0] = __uint_as_float((uint32_t)*scp << 23);
              sc[u][ng][1] = sc[u][ng][0];
            } else {
              const uint32_t two = *reinterpret_cast<const uint16_t*>(scp);
              sc[u][ng][0] = e4m3_to_f32(two & 0xffu);
              sc[u][ng][1] = e4m3_to_f32(two >> 8);
            }
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (AFMT == FP4MOE_A_BF16) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              a4[u][mb][s] = av[mb] ? *reinterpret_cast<const uint4*>(ap[mb] + blk * 64 + s * 16)
                                    : make_uint4(0, 0, 0, 0);
            }
            asc[u][mb] = 1.0f;
          } else {
            a4[u][mb][0] = av[mb] ? *reinterpret_cast<const uint4*>(ap[mb] + blk * 16)
                                  : make_uint4(0, 0, 0, 0);
            asc[u][mb] = __uint_as_float((uint32_t)(av[mb] ? asp[mb][blk] : 127) << 23);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + 4 * u >= nkc) break;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8bf b[NG];
#pragma unroll
          for (int ng = 0; ng < NG; ++ng) {
            if (WFMT == FP4MOE_W_MXFP4) {
              b[ng] = decode_mx8(word(wv[u][ng][0], s), sc[u][ng][0]);
            } else if (WFMT == FP4MOE_W_NVFP4) {
              b[ng] = decode_nv8(word(wv[u][ng][0], s), sc[u][ng][s >> 1]);
            } else {
              const uint4& h = wv[u][ng][s >> 1];
              b[ng] = decode_fp8x8(word(h, (s & 1) * 2), word(h, (s & 1) * 2 + 1));
            }
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const v8bf a = (AFMT == FP4MOE_A_BF16) ? as_bf8(a4[u][mb][s])
                                                   : decode_mx8(word(a4[u][mb][0], s), asc[u][mb]);
#pragma unroll
            for (int ng = 0; ng < NG; ++ng)
              acc[mb][ng] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[ng], acc[mb][ng], 0, 0, 0);
          }
        }
      }
    }

    // K reduction over the four waves, in wave order.
    if (wave > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave - 1][(mb * NG + ng) * 4 + i][lane] = acc[mb][ng][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ng = 0; ng < NG; ++ng)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][ng][i] += red[w][(mb * NG + ng) * 4 + i][lane];
      float cs[NG];
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        if (WFMT == FP4MOE_W_NVFP4) cs[ng] = p.w_tensor_scale[e];
        else if (WFMT == FP4MOE_W_FP8) cs[ng] = p.w_channel_scale[(int64_t)e * p.N + wrow[ng]];
        else cs[ng] = 1.0f;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + mb * 16 + g * 4 + i;
          if (r >= row_end) continue;
          if (STAGE == 1) {
            const float h = silu_mul(acc[mb][0][i] * cs[0], acc[mb][1][i] * cs[1]);
            const int64_t o = (int64_t)r * p.ldo + nb * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          } else {
#pragma unroll
            for (int ng = 0; ng < NG; ++ng) {
              const float y = acc[mb][ng][i] * cs[ng];
              const int64_t o = (int64_t)r * p.ldo + nb * 32 + ng * 16 + r16;
              p.out[o] = (uint16_t)f32_to_bf16_rne(y);
              if (p.out_f32) p.out_f32[o] = y;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// ===========================================================================
// mx family: MXFP4 activations, scaled MFMA FP4 x (FP4 | FP8)
// ===========================================================================

// Waves form a 2 x 2 grid over the workgroup tile; each wave owns WM M-blocks
// and WN weight-row blocks of 16.  Stage 1 pairs gate block j with up block
// j + WN/2 so SiLU(gate)*up is lane-local.
template <int STAGE, int WM, int WN>
__global__ __launch_bounds__(256) void mx_gemm_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BM = 2 * WM * 16;
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (WN / 2) * 16 : WN * 16;  // output columns
  constexpr int OUT_PER_WG = 2 * OUT_PER_WAVE;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int64_t wrow_bytes = p.K / 2;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const int64_t a_row_bytes = p.lda / 2, a_srow = p.lda / 32;

  for (int64_t wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
    const int tile = (int)(wi / n_nb), nb = (int)(wi - (int64_t)tile * n_nb);
    const int e = p.tiles[2 * tile], mt = p.tiles[2 * tile + 1];
    const int row0 = p.offsets[e] + mt * BM + wm * WM * 16;
    const int row_end = min(p.offsets[e + 1], p.offsets[e] + (mt + 1) * BM);
    const int col0 = nb * OUT_PER_WG + wn * OUT_PER_WAVE;   // first output column of this wave

    const uint8_t* ap[WM];
    const uint8_t* asp[WM];
    bool av[WM];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
      const int r = row0 + mb * 16 + r16;
      av[mb] = r < row_end;
      int64_t arow = r;
      if (av[mb] && p.gather) arow = p.gather[r] / p.gather_div;
      if (!av[mb]) arow = 0;
      ap[mb] = A + arow * a_row_bytes;
      asp[mb] = p.a_scale + arow * a_srow;
    }
    const uint8_t* wp[WN];
    const uint8_t* sp[WN];
#pragma unroll
    for (int nbk = 0; nbk < WN; ++nbk) {
      int wr;
      if (STAGE == 1) {
        wr = (nbk < WN / 2) ? (col0 + nbk * 16 + r16) : (p.N / 2 + col0 + (nbk - WN / 2) * 16 + r16);
      } else {
        wr = col0 + nbk * 16 + r16;
      }
      if (p.w_layout == 0) {
        const int64_t row = (int64_t)e * p.N + wr;
        wp[nbk] = p.w + row * wrow_bytes + g * 16;
        sp[nbk] = p.w_scale + row * (p.K / 32) + g;
      } else {
        const int64_t f0 = ((int64_t)e * (p.N / 16) + wr / 16) * nkc;
        wp[nbk] = p.w + f0 * 1024 + lane * 16;
        sp[nbk] = p.w_scale + ((int64_t)e * nkc * (p.N / 16) + wr / 16) * 64 + lane;
      }
    }
    const int64_t wstride = (p.w_layout == 0) ? 64 : 1024;
    const int64_t sstride = (p.w_layout == 0) ? 4 : (int64_t)(p.N / 16) * 64;

    v4f acc[WM][WN];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) acc[mb][nbk] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nkc; ++c) {
      const int blk = c * 4 + g;
      v8i af[WM];
      int as[WM];
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        uint4 v = make_uint4(0, 0, 0, 0);
        int s = 127;
        if (av[mb]) {
          v = *reinterpret_cast<const uint4*>(ap[mb] + blk * 16);
          s = asp[mb][blk];
        }
        af[mb] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        as[mb] = s;
      }
      v8i bf[WN];
      int bs[WN];
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) {
        const uint4 v = *reinterpret_cast<const uint4*>(wp[nbk] + (int64_t)c * wstride);
        bf[nbk] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        bs[nbk] = sp[nbk][(int64_t)c * sstride];
      }
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int nbk = 0; nbk < WN; ++nbk)
          acc[mb][nbk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[mb], bf[nbk], acc[mb][nbk], 4, 4, 0, as[mb], 0, bs[nbk]);
    }

    // epilogue
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + mb * 16 + g * 4 + i;
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < WN / 2; ++j) {
            const float h = silu_mul(acc[mb][j][i], acc[mb][j + WN / 2][i]);
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int nbk = 0; nbk < WN; ++nbk) {
            const float y = acc[mb][nbk][i];
            const int64_t o = (int64_t)r * p.ldo + col0 + nbk * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            if (p.out_f32) p.out_f32[o] = y;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// mx family, large tiles (block_m 128 / 256): prefill-sized expert segments.
//
// Four waves, one per SIMD, in a 2 (M) x 2 (N) grid; each wave owns WM x WN
// MFMA tiles (block_m 256: 8 x 8, a 128 x 128 sub-tile whose accumulators fill
// the accumulation registers), so the workgroup tile is block_m rows by 256
// weight rows (stage 1: 128 gate + 128 up rows, 128 output columns).  The
// activation tile of each 128-wide K chunk is staged in LDS, double buffered,
// in MFMA fragment order (one M block is one conflict-free 16-byte LDS read
// per lane); the weights are streamed straight into registers one chunk
// ahead.  Work items are split statically by XCD (workgroup i runs on XCD
// i % 8): each XCD walks a contiguous range of (tile, column block) items, so
// the column blocks of one expert tile run on one XCD and its activation tile
// stays in that XCD's L2.
template <int STAGE, int WM>
__global__ __launch_bounds__(256, 1) void mx_lds_gemm_kernel(GemmParams p) {
  constexpr int NT = 256;                           // threads
  constexpr int BM = 32 * WM;                       // tile rows (two waves in M)
  constexpr int WN = 8;                             // 16-row weight blocks per wave
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (WN / 2) * 16 : WN * 16;
  constexpr int OUT_PER_WG = 2 * OUT_PER_WAVE;
  constexpr int PIECES = BM * 4 / NT;               // 16-byte A pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 64];
  __shared__ uint8_t lds_s[2][BM * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r16 = lane & 15;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const int64_t a_row_bytes = p.lda / 2, a_srow = p.lda / 32;

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  const int64_t per = (n_work + NX - 1) / NX;
  const int64_t w_begin = (int64_t)xcd * per;
  const int64_t w_end = min(n_work, w_begin + per);

  for (int64_t wi = w_begin + slot; wi < w_end; wi += slots) {
    const int tile = (int)(wi / n_nb), nb = (int)(wi - (int64_t)tile * n_nb);
    const int e = p.tiles[2 * tile], mt = p.tiles[2 * tile + 1];
    const int tile_row0 = p.offsets[e] + mt * BM;
    const int row_end = min(p.offsets[e + 1], tile_row0 + BM);

    // A loader: piece q = tid + NT*j covers tile row q/4, block q%4 of a chunk
    const uint8_t* a_src[PIECES];
    int a_lds[PIECES];
    bool a_ok[PIECES];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int q = tid + NT * j;
      const int rr = q >> 2, b = q & 3;
      const int r = tile_row0 + rr;
      a_ok[j] = r < row_end;
      int64_t arow = 0;
      if (a_ok[j]) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      a_src[j] = A + arow * a_row_bytes + b * 16;
      a_lds[j] = (rr >> 4) * 1024 + (b * 16 + (rr & 15)) * 16;
    }
    const uint8_t* s_src = p.a_scale;
    bool s_ok = false;
    if (tid < BM) {
      const int r = tile_row0 + tid;
      s_ok = r < row_end;
      int64_t arow = 0;
      if (s_ok) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      s_src = p.a_scale + arow * a_srow;
    }
    const int s_lds = (tid >> 4) * 64 + (tid & 15);

    // B (weights): per lane, a base address plus a 32-bit offset per block;
    // chunk c of block nbk is at base + off[nbk] + c * wstride.
    const int col0 = nb * OUT_PER_WG + wn * OUT_PER_WAVE;
    const uint8_t* wbase;
    const uint8_t* sbase;
    uint32_t woff[WN], soff[WN];
    const int64_t wstride = (p.w_layout == 0) ? 64 : 1024;
    const int64_t sstride = (p.w_layout == 0) ? 4 : (int64_t)(p.N / 16) * 64;
    {
      const int wr0 = (STAGE == 1) ? col0 : col0;   // first weight row of block 0
      const int64_t e_rows = (int64_t)e * p.N;
      if (p.w_layout == 0) {
        wbase = p.w + (e_rows + wr0) * (p.K / 2) + g * 16 + (int64_t)r16 * (p.K / 2);
        sbase = p.w_scale + (e_rows + wr0) * (p.K / 32) + g + (int64_t)r16 * (p.K / 32);
      } else {
        const int64_t f0 = (e_rows / 16 + wr0 / 16) * nkc;
        wbase = p.w + f0 * 1024 + lane * 16;
        sbase = p.w_scale + ((int64_t)e * nkc * (p.N / 16) + wr0 / 16) * 64 + lane;
      }
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) {
        int dr;   // weight-row distance of block nbk from block 0
        if (STAGE == 1) dr = (nbk < WN / 2) ? nbk * 16 : p.N / 2 + (nbk - WN / 2) * 16;
        else dr = nbk * 16;
        if (p.w_layout == 0) {
          woff[nbk] = (uint32_t)((int64_t)dr * (p.K / 2));
          soff[nbk] = (uint32_t)((int64_t)dr * (p.K / 32));
        } else {
          woff[nbk] = (uint32_t)((int64_t)(dr / 16) * nkc * 1024);
          soff[nbk] = (uint32_t)((dr / 16) * 64);
        }
      }
    }

    v4f acc[WM][WN];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) acc[mb][nbk] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 a_reg[PIECES];
    uint32_t s_reg = 0x7f7f7f7fu;
    uint4 bw[WN], bw_next[WN];
    int bs[WN], bs_next[WN];

    // prologue: chunk 0
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
      a_reg[j] = a_ok[j] ? *reinterpret_cast<const uint4*>(a_src[j]) : make_uint4(0, 0, 0, 0);
    if (s_ok) s_reg = *reinterpret_cast<const uint32_t*>(s_src);
#pragma unroll
    for (int nbk = 0; nbk < WN; ++nbk) {
      bw[nbk] = *reinterpret_cast<const uint4*>(wbase + woff[nbk]);
      bs[nbk] = sbase[soff[nbk]];
    }
#pragma unroll
    for (int j = 0; j < PIECES; ++j) *reinterpret_cast<uint4*>(&lds_a[0][a_lds[j]]) = a_reg[j];
    if (tid < BM) {
#pragma unroll
      for (int b = 0; b < 4; ++b) lds_s[0][s_lds + b * 16] = (uint8_t)(s_reg >> (8 * b));
    }
    __syncthreads();

    for (int c = 0; c < nkc; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < nkc;
      // next chunk's loads go out before this chunk's MFMAs
      if (more) {
#pragma unroll
        for (int j = 0; j < PIECES; ++j)
          a_reg[j] = a_ok[j] ? *reinterpret_cast<const uint4*>(a_src[j] + (int64_t)(c + 1) * 64)
                             : make_uint4(0, 0, 0, 0);
        if (s_ok) s_reg = *reinterpret_cast<const uint32_t*>(s_src + (c + 1) * 4);
        const uint8_t* wnext = wbase + (int64_t)(c + 1) * wstride;
        const uint8_t* snext = sbase + (int64_t)(c + 1) * sstride;
#pragma unroll
        for (int nbk = 0; nbk < WN; ++nbk) {
          bw_next[nbk] = *reinterpret_cast<const uint4*>(wnext + woff[nbk]);
          bs_next[nbk] = snext[soff[nbk]];
        }
      }
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const int mblk = wm * WM + mb;
        const uint4 av = *reinterpret_cast<const uint4*>(&lds_a[buf][mblk * 1024 + lane * 16]);
        const int as = lds_s[buf][mblk * 64 + lane];
        const v8i af = v8i{(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
#pragma unroll
        for (int nbk = 0; nbk < WN; ++nbk) {
          const v8i bf = v8i{(int)bw[nbk].x, (int)bw[nbk].y, (int)bw[nbk].z, (int)bw[nbk].w,
                             0, 0, 0, 0};
          acc[mb][nbk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf, acc[mb][nbk], 4, 4, 0, as, 0, bs[nbk]);
        }
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < PIECES; ++j)
          *reinterpret_cast<uint4*>(&lds_a[buf ^ 1][a_lds[j]]) = a_reg[j];
        if (tid < BM) {
#pragma unroll
          for (int b = 0; b < 4; ++b) lds_s[buf ^ 1][s_lds + b * 16] = (uint8_t)(s_reg >> (8 * b));
        }
#pragma unroll
        for (int nbk = 0; nbk < WN; ++nbk) {
          bw[nbk] = bw_next[nbk];
          bs[nbk] = bs_next[nbk];
        }
      }
      __syncthreads();
    }

    // epilogue
    const int wrow0 = tile_row0 + wm * WM * 16;
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wrow0 + mb * 16 + g * 4 + i;
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < WN / 2; ++j) {
            const float h = silu_mul(acc[mb][j][i], acc[mb][j + WN / 2][i]);
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int nbk = 0; nbk < WN; ++nbk) {
            const float y = acc[mb][nbk][i];
            const int64_t o = (int64_t)r * p.ldo + col0 + nbk * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            if (p.out_f32) p.out_f32[o] = y;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// mx family, large tiles, fragment-major weights: LDS-DMA pipeline.
//
// Same workgroup tile and wave grid as mx_lds_gemm_kernel, but every operand
// of a 128-wide K chunk -- activation codes and scales, weight fragments and
// scales -- is copied global -> LDS by the LDS-DMA form of the global load
// (no staging registers), into a ring of S stages.  Each wave issues D DMA
// instructions per chunk; before computing chunk c it waits until at most
// D * (chunks issued after c) of its loads are outstanding (vector-memory
// loads retire in issue order), then a workgroup barrier makes every wave's
// copies visible.  The DMA for chunk c+S-1 is issued right after that
// barrier into the stage computed in the previous step, so S-1 chunks are in
// flight while one is computed.  The loads are issued from inline assembly so
// that the compiler does not drain the whole ring at every barrier.
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

template <int STAGE, int WM>
__global__ __launch_bounds__(256, 1) void mx_dma_gemm_kernel(GemmParams p) {
  constexpr int S = 4;                              // pipeline stages
  constexpr int BM = 32 * WM;
  constexpr int WN = 8;
  constexpr int MBLK = BM / 16;                     // M blocks per tile
  constexpr int A_MB_PER_WAVE = MBLK / 4;
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (WN / 2) * 16 : WN * 16;
  constexpr int OUT_PER_WG = 2 * OUT_PER_WAVE;
  constexpr int OFF_AS = BM * 64;                   // A codes: [MBLK][64 lanes][16 B]
  constexpr int OFF_B = OFF_AS + BM * 4;            // A scales: [row][4 blocks]
  constexpr int OFF_BS = OFF_B + 16 * 1024;         // B codes: [16 groups][64 lanes][16 B]
  constexpr int STAGE_BYTES = OFF_BS + 16 * 64;     // B scales: [16 groups][64 lanes]
  constexpr int D = A_MB_PER_WAVE + 1 + 4 + 1;      // DMA instructions per wave per chunk
  static_assert(D * (S - 2) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r16 = lane & 15;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int G = p.N / 16;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const int64_t a_row_bytes = p.lda / 2, a_srow = p.lda / 32;
  const uint32_t smem_base = lds_offset(smem);

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  const int64_t per = (n_work + NX - 1) / NX;
  const int64_t w_begin = (int64_t)xcd * per;
  const int64_t w_end = min(n_work, w_begin + per);

  for (int64_t wi = w_begin + slot; wi < w_end; wi += slots) {
    // Items of one expert are ordered (column block, M tile): the M tiles that
    // share a weight slice run side by side on one XCD, so the slice is read
    // from HBM once and from L2 for the other tiles.
    const int any_tile = (int)(wi / n_nb);
    const int e = p.tiles[2 * any_tile];
    const int t0 = any_tile - p.tiles[2 * any_tile + 1];
    const int m_tiles = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    const int local = (int)(wi - (int64_t)t0 * n_nb);
    const int nb = local / m_tiles, mt = local - nb * m_tiles;
    const int tile_row0 = p.offsets[e] + mt * BM;
    const int row_end = min(p.offsets[e + 1], tile_row0 + BM);

    // DMA sources of this wave: uniform 64-bit bases plus 32-bit lane offsets;
    // rows past the segment read row 0.
    uint32_t a_off[A_MB_PER_WAVE];
#pragma unroll
    for (int j = 0; j < A_MB_PER_WAVE; ++j) {
      const int r = tile_row0 + (wave * A_MB_PER_WAVE + j) * 16 + r16;
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      a_off[j] = (uint32_t)(arow * a_row_bytes) + g * 16;
    }
    uint32_t as_off;
    {
      const int r = tile_row0 + (wave % (BM / 64)) * 64 + lane;   // BM=128: waves 2,3 repeat 0,1
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      as_off = (uint32_t)(arow * a_srow);
    }
    // the workgroup's 16 weight groups: stage 1 gate 0..7 then up 0..7;
    // wave w copies groups 4w..4w+3 (one run of 4 for the scales)
    const int grp0 = (STAGE == 1) ? ((wave < 2) ? nb * 8 + wave * 4 : G / 2 + nb * 8 + (wave - 2) * 4)
                                  : nb * 16 + wave * 4;
    const uint8_t* b_base = p.w + ((int64_t)e * G + grp0) * nkc * 1024;
    const uint32_t b_lane = lane * 16;
    const uint8_t* bs_base = p.w_scale + ((int64_t)e * nkc * G + grp0) * 64;
    const uint32_t bs_lane = lane * 4;
    const uint32_t lds_wave = smem_base + (uint32_t)(wave * 0);   // uniform base

    auto issue = [&](int c) {
      const uint32_t st = lds_wave + (uint32_t)((c % S) * STAGE_BYTES);
#pragma unroll
      for (int j = 0; j < A_MB_PER_WAVE; ++j)
        dma_b128(A + a_off[j] + (int64_t)c * 64, st + (wave * A_MB_PER_WAVE + j) * 1024);
      dma_b32(p.a_scale + as_off + c * 4, st + OFF_AS + (wave % (BM / 64)) * 256);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dma_b128(b_base + ((int64_t)q * nkc + c) * 1024 + b_lane, st + OFF_B + (wave * 4 + q) * 1024);
      dma_b32(bs_base + (int64_t)c * G * 64 + bs_lane, st + OFF_BS + wave * 256);
    };

    v4f acc[WM][WN];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) acc[mb][nbk] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < S - 1 && c < nkc; ++c) issue(c);

    // per-lane LDS read bases within a stage; fragments sit at constant offsets
    const int a_lds = wm * WM * 1024 + lane * 16;
    const int as_lds = OFF_AS + wm * WM * 64 + r16 * 4 + g;
    const int b_lds = OFF_B + ((STAGE == 1) ? wn * 4 : wn * 8) * 1024 + lane * 16;
    const int bs_lds = OFF_BS + ((STAGE == 1) ? wn * 4 : wn * 8) * 64 + lane;

    for (int c = 0; c < nkc; ++c) {
      const int newer = min(S - 2, nkc - 1 - c);
      if (newer >= 2) wait_vmcnt<2 * D>();
      else if (newer == 1) wait_vmcnt<D>();
      else wait_vmcnt<0>();
      wg_barrier();
      if (c + S - 1 < nkc) issue(c + S - 1);

      const uint8_t* st = smem + (c % S) * STAGE_BYTES;
      v8i bf[WN];
      int bsc[WN];
#pragma unroll
      for (int nbk = 0; nbk < WN; ++nbk) {
        // stage 1: gate blocks 0..3 at groups wn*4+q, up blocks at 8+wn*4+q
        const int jo = (STAGE == 1) ? ((nbk < WN / 2) ? nbk : 8 + (nbk - WN / 2)) : nbk;
        const uint4 v = *reinterpret_cast<const uint4*>(st + b_lds + jo * 1024);
        bf[nbk] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        bsc[nbk] = st[bs_lds + jo * 64];
      }
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const uint4 av = *reinterpret_cast<const uint4*>(st + a_lds + mb * 1024);
        const int as = st[as_lds + mb * 64];
        const v8i af = v8i{(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
#pragma unroll
        for (int nbk = 0; nbk < WN; ++nbk)
          acc[mb][nbk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[nbk], acc[mb][nbk], 4, 4, 0, as, 0, bsc[nbk]);
      }
    }
    wg_barrier();   // every wave is done with the ring before the next item refills it

    // epilogue
    const int col0 = nb * OUT_PER_WG + wn * OUT_PER_WAVE;
    const int wrow0 = tile_row0 + wm * WM * 16;
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wrow0 + mb * 16 + g * 4 + i;
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < WN / 2; ++j) {
            const float h = silu_mul(acc[mb][j][i], acc[mb][j + WN / 2][i]);
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int nbk = 0; nbk < WN; ++nbk) {
            const float y = acc[mb][nbk][i];
            const int64_t o = (int64_t)r * p.ldo + col0 + nbk * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            if (p.out_f32) p.out_f32[o] = y;
          }
        }
      }
      // keep the scheduler from pulling every accumulator out at once
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ===========================================================================
// dispatch
// ===========================================================================

static int g_num_cus = 0;

static int grid_cap() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus = n;
  }
  return g_num_cus * 8;
}

template <int WFMT, int AFMT, int STAGE>
static void launch_dq(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int n_nb = (STAGE == 1) ? (p.N / 2) / 16 : p.N / 32;
  int64_t work = (int64_t)max_tiles * n_nb;
  const int grid = (int)(work < grid_cap() ? (work < 1 ? 1 : work) : grid_cap());
  switch (p.block_m) {
    case 16: hipLaunchKernelGGL((dq_gemm_kernel<WFMT, AFMT, STAGE, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 32: hipLaunchKernelGGL((dq_gemm_kernel<WFMT, AFMT, STAGE, 2>), dim3(grid), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((dq_gemm_kernel<WFMT, AFMT, STAGE, 4>), dim3(grid), dim3(256), 0, s, p); break;
  }
}

template <int WFMT, int AFMT>
static void launch_dq_stage(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  if (stage == 1) launch_dq<WFMT, AFMT, 1>(p, max_tiles, s);
  else launch_dq<WFMT, AFMT, 2>(p, max_tiles, s);
}

template <int STAGE, int WM>
static void launch_mx_wm(const GemmParams& p, int max_tiles, hipStream_t s) {
  constexpr int WN = 4;
  const int out_per_wg = 2 * ((STAGE == 1) ? (WN / 2) * 16 : WN * 16);
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  const int grid = (int)(work < grid_cap() ? (work < 1 ? 1 : work) : grid_cap());
  hipLaunchKernelGGL((mx_gemm_kernel<STAGE, WM, WN>), dim3(grid), dim3(256), 0, s, p);
}

template <int STAGE, int WM>
static void launch_mx_lds(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int out_per_wg = (STAGE == 1) ? 128 : 256;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  int cap = grid_cap() / 8;              // one workgroup (four waves) per CU
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((mx_lds_gemm_kernel<STAGE, WM>), dim3(grid), dim3(256), 0, s, p);
}

template <int STAGE, int WM>
static void launch_mx_dma(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int out_per_wg = (STAGE == 1) ? 128 : 256;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  int cap = grid_cap() / 8;              // one workgroup (four waves) per CU
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((mx_dma_gemm_kernel<STAGE, WM>), dim3(grid), dim3(256), 0, s, p);
}

template <int STAGE>
static void launch_mx(const GemmParams& p, int max_tiles, hipStream_t s) {
  const bool frag = p.w_layout == FP4MOE_LAYOUT_FRAGMENT;
  switch (p.block_m) {
    case 32: launch_mx_wm<STAGE, 1>(p, max_tiles, s); break;
    case 64: launch_mx_wm<STAGE, 2>(p, max_tiles, s); break;
    case 128:
      if (frag) launch_mx_dma<STAGE, 4>(p, max_tiles, s);
      else launch_mx_lds<STAGE, 4>(p, max_tiles, s);
      break;
    default: launch_mx_lds<STAGE, 8>(p, max_tiles, s); break;
  }
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int fp4_grouped_gemm(const fp4moe_gemm_args* a, void* stream) {
  FP4MOE_REQUIRE(a, "fp4_grouped_gemm: null args");
  FP4MOE_REQUIRE(a->stage == 1 || a->stage == 2, "fp4_grouped_gemm: stage=%d", a->stage);
  const bool mx = a->afmt == FP4MOE_A_MXFP4 && a->wfmt == FP4MOE_W_MXFP4;
  const bool dq = !mx;
  FP4MOE_REQUIRE(a->afmt == FP4MOE_A_BF16 || a->afmt == FP4MOE_A_MXFP4,
                 "fp4_grouped_gemm: afmt=%d", a->afmt);
  FP4MOE_REQUIRE(a->wfmt == FP4MOE_W_MXFP4 || a->wfmt == FP4MOE_W_NVFP4 || a->wfmt == FP4MOE_W_FP8,
                 "fp4_grouped_gemm: wfmt=%d", a->wfmt);
  FP4MOE_REQUIRE(!(a->wfmt == FP4MOE_W_NVFP4 && a->afmt == FP4MOE_A_MXFP4),
                 "fp4_grouped_gemm: NVFP4 weights take bf16 activations (nvfp4_qdq output)");
  FP4MOE_REQUIRE(a->K > 0 && a->K % 128 == 0, "fp4_grouped_gemm: K=%d not a multiple of 128", a->K);
  FP4MOE_REQUIRE(a->N > 0 && a->N % 32 == 0 && (a->stage == 2 || a->N % 64 == 0),
                 "fp4_grouped_gemm: N=%d (stage %d)", a->N, a->stage);
  if (dq) {
    FP4MOE_REQUIRE(a->block_m == 16 || a->block_m == 32 || a->block_m == 64,
                   "fp4_grouped_gemm: block_m=%d not in {16,32,64} for this format pair",
                   a->block_m);
  } else {
    FP4MOE_REQUIRE(a->block_m == 32 || a->block_m == 64 || a->block_m == 128 || a->block_m == 256,
                   "fp4_grouped_gemm: block_m=%d not in {32,64,128,256} for MXFP4 x MXFP4",
                   a->block_m);
    const bool big = a->block_m >= 128;
    const int out_per_wg = (a->stage == 1 ? 64 : 128) * (big ? 2 : 1);
    const int n_out = a->stage == 1 ? a->N / 2 : a->N;
    FP4MOE_REQUIRE(n_out % out_per_wg == 0,
                   "fp4_grouped_gemm: output width %d not a multiple of %d", n_out, out_per_wg);
  }
  FP4MOE_REQUIRE(a->n_experts >= 1 && a->max_rows >= 0 && a->max_tiles >= 0,
                 "fp4_grouped_gemm: n_experts=%d max_rows=%d max_tiles=%d", a->n_experts,
                 a->max_rows, a->max_tiles);
  FP4MOE_REQUIRE(a->gather_div >= 1, "fp4_grouped_gemm: gather_div=%d", a->gather_div);
  FP4MOE_REQUIRE(a->w_layout == FP4MOE_LAYOUT_ROWMAJOR || a->w_layout == FP4MOE_LAYOUT_FRAGMENT,
                 "fp4_grouped_gemm: w_layout=%d", a->w_layout);
  FP4MOE_REQUIRE(a->w_layout == FP4MOE_LAYOUT_ROWMAJOR || a->N % 16 == 0,
                 "fp4_grouped_gemm: fragment layout needs N %% 16 == 0");
  const int n_out = a->stage == 1 ? a->N / 2 : a->N;
  FP4MOE_REQUIRE(a->ldo >= n_out, "fp4_grouped_gemm: ldo=%lld < %d", (long long)a->ldo, n_out);
  FP4MOE_REQUIRE(a->lda >= a->K && a->lda % 32 == 0, "fp4_grouped_gemm: lda=%lld",
                 (long long)a->lda);
  if (a->max_tiles == 0 || a->max_rows == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(a->w && a->a && a->expert_offsets && a->tiles && a->n_tiles && a->out,
                 "fp4_grouped_gemm: null pointer");
  FP4MOE_REQUIRE(a->wfmt == FP4MOE_W_FP8 || a->w_scale, "fp4_grouped_gemm: w_scale is null");
  FP4MOE_REQUIRE(a->wfmt != FP4MOE_W_NVFP4 || a->w_tensor_scale,
                 "fp4_grouped_gemm: NVFP4 needs w_tensor_scale");
  FP4MOE_REQUIRE(a->wfmt != FP4MOE_W_FP8 || a->w_channel_scale,
                 "fp4_grouped_gemm: FP8 needs w_channel_scale");
  FP4MOE_REQUIRE(a->afmt != FP4MOE_A_MXFP4 || a->a_scale,
                 "fp4_grouped_gemm: MXFP4 activations need a_scale");
  FP4MOE_REQUIRE(((uintptr_t)a->w & 15) == 0 && ((uintptr_t)a->a & 15) == 0,
                 "fp4_grouped_gemm: w and a must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();

  GemmParams p;
  p.N = a->N;
  p.K = a->K;
  p.n_experts = a->n_experts;
  p.block_m = a->block_m;
  p.gather_div = a->gather_div;
  p.w_layout = a->w_layout;
  p.lda = a->lda;
  p.ldo = a->ldo;
  p.w = a->w;
  p.w_scale = a->w_scale;
  p.w_tensor_scale = a->w_tensor_scale;
  p.w_channel_scale = a->w_channel_scale;
  p.a = a->a;
  p.a_scale = a->a_scale;
  p.gather = a->a_row_gather;
  p.offsets = a->expert_offsets;
  p.tiles = a->tiles;
  p.n_tiles = a->n_tiles;
  p.out = a->out;
  p.out_f32 = a->out_f32;
  hipStream_t s = as_stream(stream);
  const int mt = a->max_tiles;
  const int st = a->stage;
  if (mx) {
    if (st == 1) launch_mx<1>(p, mt, s);
    else launch_mx<2>(p, mt, s);
  } else if (a->afmt == FP4MOE_A_BF16) {
    if (a->wfmt == FP4MOE_W_MXFP4) launch_dq_stage<FP4MOE_W_MXFP4, FP4MOE_A_BF16>(p, st, mt, s);
    else if (a->wfmt == FP4MOE_W_NVFP4) launch_dq_stage<FP4MOE_W_NVFP4, FP4MOE_A_BF16>(p, st, mt, s);
    else launch_dq_stage<FP4MOE_W_FP8, FP4MOE_A_BF16>(p, st, mt, s);
  } else {
    launch_dq_stage<FP4MOE_W_FP8, FP4MOE_A_MXFP4>(p, st, mt, s);
  }
  return check_launch("fp4_grouped_gemm");
}
