// One work item of the dq family of fp4_grouped_gemm (bf16 or MXFP4-decoded
// activations times MXFP4 / NVFP4 / FP8 weights decoded to bf16 in registers,
// bf16 MFMA), shared by the dq kernel and the fused decode kernel.
//
// A work item is one tile of MB*16 rows of an expert segment times NG 16-row
// weight groups (stage 1: NG/2 gate groups and the NG/2 up groups of the same
// output columns, so SiLU(gate)*up is lane-local).  The NW waves of a
// workgroup take the K chunks of the item round-robin and add their partial
// sums through LDS.  Each step of a wave issues the loads of U of its chunks
// before the first MFMA.  Weight bytes are read exactly once per call, so
// they are fetched with non-temporal (streaming) loads; the activation rows,
// which every work item of a tile re-reads, use ordinary cached loads.  On the
// decode stream the streaming form measured about 13% faster than cached
// loads.
//
// The tile list, expert offsets and row gather of `p` may point to LDS (the
// fused decode kernel keeps its own permutation there).
#pragma once

#include "gemm_common.h"

namespace fp4moe {

__device__ __forceinline__ uint4 stream_load16(const uint8_t* ptr) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u*>(ptr)));
}

// Output columns of one work item.
template <int STAGE, int NG>
constexpr int dq_out_cols() { return (STAGE == 1) ? (NG / 2) * 16 : NG * 16; }

// Work item wi = tile * n_nb + column block of stage STAGE; every thread of
// the workgroup calls it.  red: the LDS reduction buffer [NW - 1][MB*NG*4][64].
// Ends with a workgroup barrier.
template <int WFMT, int AFMT, int STAGE, int MB, int NG, int U, int NW>
__device__ __forceinline__ void dq_item(const GemmParams& p, int64_t wi,
                                        float (*red)[MB * NG * 4][64]) {
  static_assert(STAGE == 2 || NG % 2 == 0, "stage 1 pairs gate and up groups");
  constexpr int NGH = NG / 2;
  constexpr int OUT_COLS = dq_out_cols<STAGE, NG>();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int BM = MB * 16;
  const int n_nb = ((STAGE == 1) ? p.N / 2 : p.N) / OUT_COLS;
  const int nkc = p.K / 128;
  const int64_t wrow_bytes = (WFMT == FP4MOE_W_FP8) ? p.K : p.K / 2;
  const int64_t srow_bytes = (WFMT == FP4MOE_W_MXFP4) ? p.K / 32 : p.K / 16;
  const int tile = (int)(wi / n_nb), nb = (int)(wi - (int64_t)tile * n_nb);
  const int e = p.tiles[2 * tile], mt = p.tiles[2 * tile + 1];
  const int row0 = p.offsets[e] + mt * BM;
  const int row_end = min(p.offsets[e + 1], row0 + BM);

  // Weight code / scale addresses = per-group base (wave-uniform, scalar
  // registers) + per-lane offset (one 32-bit register, shared by all groups
  // and chunks) + chunk * stride (uniform), for the row-major or the
  // fragment-major layout.
  int64_t w_base[NG], s_base[NG];
  int wrow0[NG];
  uint32_t w_lane, s_lane;
  int64_t wstride, sstride, whalf;
  constexpr int SPB = (WFMT == FP4MOE_W_MXFP4) ? 1 : 2;   // scale bytes per 32-block
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    int wr;   // first weight row of the group
    if (STAGE == 1)
      wr = (ng < NGH) ? nb * OUT_COLS + ng * 16 : p.N / 2 + nb * OUT_COLS + (ng - NGH) * 16;
    else
      wr = nb * OUT_COLS + ng * 16;
    wrow0[ng] = wr;
    if (p.w_layout == 0) {
      const int64_t row = (int64_t)e * p.N + wr;
      w_base[ng] = row * wrow_bytes;
      s_base[ng] = row * srow_bytes;
    } else {
      const int64_t grp = (int64_t)e * (p.N / 16) + wr / 16;
      w_base[ng] = grp * nkc * ((WFMT == FP4MOE_W_FP8) ? 2048 : 1024);
      // scales are chunk-major: (e*C + c)*G + group
      s_base[ng] = ((int64_t)e * nkc * (p.N / 16) + wr / 16) * (64 * SPB);
    }
  }
  if (p.w_layout == 0) {
    w_lane = (uint32_t)(r16 * wrow_bytes + g * (WFMT == FP4MOE_W_FP8 ? 32 : 16));
    s_lane = (uint32_t)(r16 * srow_bytes + g * SPB);
    wstride = (WFMT == FP4MOE_W_FP8) ? 128 : 64;
    whalf = 16;
    sstride = 4 * SPB;
  } else {
    w_lane = (uint32_t)(lane * 16);
    s_lane = (uint32_t)(lane * SPB);
    wstride = (WFMT == FP4MOE_W_FP8) ? 2048 : 1024;
    whalf = 1024;
    sstride = (int64_t)(p.N / 16) * (64 * SPB);
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

  for (int c0 = wave; c0 < nkc; c0 += NW * U) {
    uint4 wv[U][NG][2];
    float sc[U][NG][2];
    uint4 a4[U][MB][4];
    float asc[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + NW * u;
      if (c >= nkc) break;
      const int blk = c * 4 + g;
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const uint8_t* wc = (p.w + (w_base[ng] + c * wstride)) + w_lane;
        if (WFMT == FP4MOE_W_FP8) {
          wv[u][ng][0] = stream_load16(wc);
          wv[u][ng][1] = stream_load16(wc + whalf);
          sc[u][ng][0] = sc[u][ng][1] = 1.0f;
        } else {
          wv[u][ng][0] = stream_load16(wc);
          wv[u][ng][1] = wv[u][ng][0];
          const uint8_t* scp = (p.w_scale + (s_base[ng] + c * sstride)) + s_lane;
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
      if (c0 + NW * u >= nkc) break;
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

  // K reduction over the NW waves, in wave order.
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
    for (int w = 0; w < NW - 1; ++w)
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
      else if (WFMT == FP4MOE_W_FP8) cs[ng] = p.w_channel_scale[(int64_t)e * p.N + wrow0[ng] + r16];
      else cs[ng] = 1.0f;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + mb * 16 + g * 4 + i;
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < NGH; ++j) {
            const float h = silu_mul(acc[mb][j][i] * cs[j], acc[mb][j + NGH][i] * cs[j + NGH]);
            const int64_t o = (int64_t)r * p.ldo + nb * OUT_COLS + j * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int ng = 0; ng < NG; ++ng) {
            const float y = acc[mb][ng][i] * cs[ng];
            const int64_t o = (int64_t)r * p.ldo + nb * OUT_COLS + ng * 16 + r16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            if (p.out_f32) p.out_f32[o] = y;
          }
        }
      }
    }
  }
  __syncthreads();
}

}  // namespace fp4moe
