// fp4_grouped_gemm, dq family, tiled variant for 64-row tiles (prefill-sized
// expert segments with bf16 MFMA): MXFP4 / NVFP4 / FP8 weights decoded to
// bf16 in registers, bf16 or MXFP4 activations shared by the whole workgroup
// through LDS.
//
// [NVFP4] "Memory Management": dequantization is fused into the GEMM tile, no
// bf16 weight buffer exists in memory.  [ATOM] "When Is the Scale Applied?":
// the block scale is absorbed while decoding the weight, before the MFMA.
//
// Workgroup: NW waves, a tile of 64 rows (four 16-row M blocks) by NW x NGW
// weight groups of 16 rows; wave w owns NGW groups (stage 1: NGW/2 gate
// groups and the up groups of the same output columns) for all 64 rows and
// the whole K, so every weight element is decoded once per workgroup and no
// cross-wave reduction is needed.  Every operand of a 128-wide K chunk --
// activation fragments, weight fragments, block scales -- is copied global ->
// LDS by the LDS-DMA form of the load into a ring of S stages (the same ring
// protocol as the scaled-FP4 kernel).
//
// K order inside a chunk.  The 16x16x32 bf16 MFMA takes, in lane l, eight K
// values of row l % 16.  Any assignment of K indices to (lane group, element)
// works as long as both operands use it, so K step t of lane l takes elements
// 8t..8t+7 of 32-element block l / 16: for the weights that is dword t of the
// lane's own 16-byte fragment piece (no cross-lane traffic), and the
// activation fragments in LDS are laid out to match.  (A 32x32x16 form with
// eight waves measured slower here: this kernel is bound by the weight decode
// and the copies, not by the MFMA rate.)
#include "gemm_common.h"

namespace fp4moe {

template <int WFMT, int AFMT, int STAGE, int S, int NGW, int NW>
__global__ __launch_bounds__(64 * NW, 1) void dqt_gemm_kernel(GemmParams p) {
  constexpr int MB = 4, BM = 64;                      // 16-row M blocks per tile
  constexpr int NG = NW * NGW;                        // weight groups per tile
  constexpr int RUN = NGW / 2;                        // groups per contiguous run (gate | up)
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (NGW / 2) * 16 : NGW * 16;
  constexpr int OUT_PER_WG = NW * OUT_PER_WAVE;
  constexpr bool AMX = AFMT == FP4MOE_A_MXFP4;
  constexpr bool AF16 = AFMT == FP4MOE_A_F16;           // f16 activations, NVFP4 weights
  static_assert(!AF16 || (WFMT == FP4MOE_W_NVFP4 && NGW == 4), "f16 path: NVFP4, 4 groups");
  constexpr bool W8 = WFMT == FP4MOE_W_FP8;
  constexpr int WFRAG = W8 ? 2048 : 1024;             // one 16-row x 128-K weight fragment
  constexpr int SPB = (WFMT == FP4MOE_W_MXFP4) ? 1 : 2;   // scale bytes per lane per group
  // stage layout
  constexpr int A_BYTES = AMX ? BM * 64 : BM * 256;   // MXFP4 codes | bf16 values
  constexpr int OFF_AS = A_BYTES;                     // MXFP4 activation scales [row][4]
  constexpr int OFF_B = OFF_AS + (AMX ? BM * 4 : 0);
  constexpr int RUN_SB = RUN * 64 * SPB;              // scale bytes of one run per chunk
  constexpr int SDMA = RUN_SB > 256 ? RUN_SB / 256 : 1;   // dword copies per run
  constexpr int RS = SDMA * 256;                      // LDS slot of one run's scales
  constexpr int OFF_BS = OFF_B + NG * WFRAG;          // weight scales: [wave][run][RS]
  constexpr int STAGE_BYTES = OFF_BS + (W8 ? 0 : NW * 2 * RS);
  constexpr int DA = AMX ? 2 : 16 / NW;               // activation copies per wave per chunk
  static_assert(!AMX || NW == 4, "MXFP4 activations: four waves");
  constexpr int D = DA + NGW * (W8 ? 2 : 1) + (W8 ? 0 : 2 * SDMA);
  static_assert(RUN_SB >= 256 || RUN_SB == 128, "scale run copy");
  static_assert(D * (S - 2) <= 63, "vmcnt range");
  static_assert(S >= 3 && S * STAGE_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int G = p.N / 16;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const uint32_t smem_base = lds_offset(smem);

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  const int64_t per = (n_work + NX - 1) / NX;
  const int64_t w_begin = (int64_t)xcd * per;
  const int64_t w_end = min(n_work, w_begin + per);

  for (int64_t wi = w_begin + slot; wi < w_end; wi += slots) {
    // (column block, M tile) order inside an expert: M tiles sharing a
    // weight slice run side by side on one XCD
    const int any_tile = (int)(wi / n_nb);
    const int e = p.tiles[2 * any_tile];
    const int t0 = any_tile - p.tiles[2 * any_tile + 1];
    const int m_tiles = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    const int local = (int)(wi - (int64_t)t0 * n_nb);
    const int nb = local / m_tiles, mt = local - nb * m_tiles;
    const int tile_row0 = p.offsets[e] + mt * BM;
    const int row_end = min(p.offsets[e + 1], tile_row0 + BM);

    // activation copies of this wave: bf16 the 16 / NW fragments (M block,
    // K block) from wave * 16 / NW on, all of M block wave * 4 / NW; MXFP4
    // (four waves) the codes of M block `wave`, plus one copy of the tile's
    // 64 scale rows
    int64_t a_src;
    {
      const int r = tile_row0 + (AMX ? wave : wave * 4 / NW) * 16 + r16;
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      a_src = AMX ? arow * (p.lda / 2) + g * 16 : arow * p.lda * 2 + g * 16;
    }
    int64_t as_src = 0;
    if (AMX) {
      const int r = tile_row0 + lane;
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      as_src = arow * (p.lda / 32);
    }
    // this wave's weight groups: run 0 = q < RUN, run 1 = q >= RUN (stage 1:
    // gate run, up run), each a contiguous run of groups in the tensor
    int grp_run[2];
    if (STAGE == 1) {
      grp_run[0] = nb * (NG / 2) + wave * RUN;
      grp_run[1] = G / 2 + nb * (NG / 2) + wave * RUN;
    } else {
      grp_run[0] = nb * NG + wave * NGW;
      grp_run[1] = grp_run[0] + RUN;
    }
    const int64_t w_run0 = ((int64_t)e * G + grp_run[0]) * nkc * WFRAG;
    const int64_t w_run1 = ((int64_t)e * G + grp_run[1]) * nkc * WFRAG;
    const int64_t s_run0 = ((int64_t)e * nkc * G + grp_run[0]) * (64 * SPB);
    const int64_t s_run1 = ((int64_t)e * nkc * G + grp_run[1]) * (64 * SPB);
    // scale run copy: 256-byte dword copies; a 128-byte run (MX, 2 groups)
    // has lanes 32..63 repeat 0..31
    const uint32_t bs_lane = (RUN_SB == 128) ? (lane & 31) * 4 : lane * 4;

    auto issue = [&](int c) {
      const uint32_t st = smem_base + (uint32_t)((c % S) * STAGE_BYTES);
      if (AMX) {
        dma_b128(A + a_src + (int64_t)c * 64, st + wave * 1024);
        dma_b32(p.a_scale + as_src + (int64_t)c * 4, st + OFF_AS);
      } else {
#pragma unroll
        for (int blk = 0; blk < DA; ++blk) {
          const int idx = wave * DA + blk;              // fragment (M block idx / 4, K block idx % 4)
          dma_b128(A + a_src + (int64_t)c * 256 + (idx % 4) * 64, st + idx * 1024);
        }
      }
#pragma unroll
      for (int q = 0; q < NGW; ++q) {
        const int64_t src = ((q < RUN) ? w_run0 : w_run1) + ((int64_t)(q % RUN) * nkc + c) * WFRAG;
        dma_b128(p.w + src + lane * 16, st + OFF_B + (wave * NGW + q) * WFRAG);
        if (W8) dma_b128(p.w + src + 1024 + lane * 16, st + OFF_B + (wave * NGW + q) * WFRAG + 1024);
      }
      if (!W8) {
        const int64_t sstride = (int64_t)c * G * (64 * SPB);
#pragma unroll
        for (int d = 0; d < SDMA; ++d) {
          dma_b32(p.w_scale + s_run0 + sstride + d * 256 + bs_lane, st + OFF_BS + (wave * 2) * RS + d * 256);
          dma_b32(p.w_scale + s_run1 + sstride + d * 256 + bs_lane, st + OFF_BS + (wave * 2 + 1) * RS + d * 256);
        }
      }
    };

    v4f acc[MB][NGW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < NGW; ++q) acc[mb][q] = v4f{0.f, 0.f, 0.f, 0.f};
    // f16 path: 32x32 tiles, [32-row M block][32 weight rows = 2 groups]
    v16f acc2[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc2[i][j] = v16f{};

    for (int c = 0; c < S - 1 && c < nkc; ++c) issue(c);
    for (int c = 0; c < nkc; ++c) {
      wait_chunks<D, S - 2>(min(S - 2, nkc - 1 - c));
      wait_lgkm0();   // this wave's reads of chunk c-1 are complete: its stage is refilled next
      wg_barrier();
      if (c + S - 1 < nkc) issue(c + S - 1);

      const uint8_t* st = smem + (c % S) * STAGE_BYTES;
      if constexpr (AF16) {
        // 32x32x16 f16 MFMA.  K step u (0..7) of lane half hh = l/32 takes
        // elements 16*hh + 8*(u%2) .. +7 of 32-element block u/2: for the
        // weights, dword 2*hh + u%2 of fragment piece (l%16) + 16*(u/2) of
        // group 2*nb2 + (l%32)/16 -- one NVFP4 block per (u/2, hh), so one
        // scale -- and for the activations the matching 8 values of row
        // l%32 of M block mb2.
        const int l32 = lane & 31, hh = lane >> 5;
        // every LDS read of the chunk first (their latencies overlap), then
        // the decode of block kb + 1 runs under the MFMAs of block kb
        uint2 wd[4][2];
        uint32_t sbyte[4][2];
        v8h av[8][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int nb2 = 0; nb2 < 2; ++nb2) {
            const int q = 2 * nb2 + (l32 >> 4);
            const int piece = (l32 & 15) + 16 * kb;
            wd[kb][nb2] = *reinterpret_cast<const uint2*>(
                st + OFF_B + (wave * NGW + q) * WFRAG + piece * 16 + 8 * hh);
            sbyte[kb][nb2] =
                st[OFF_BS + (wave * 2 + q / RUN) * RS + (q % RUN) * 128 + piece * 2 + hh];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int mb2 = 0; mb2 < 2; ++mb2)
            av[u][mb2] = *reinterpret_cast<const v8h*>(
                st + ((2 * mb2 + (l32 >> 4)) * 4 + (u >> 1)) * 1024 +
                ((l32 & 15) + 16 * (2 * hh + (u & 1))) * 16);
        // keep the reads here: the compiler would otherwise sink each one to
        // its first use and expose the LDS latency once per K step
        asm volatile("" : "+v"(av[0][0]), "+v"(av[0][1]), "+v"(av[1][0]), "+v"(av[1][1]),
                     "+v"(av[2][0]), "+v"(av[2][1]), "+v"(av[3][0]), "+v"(av[3][1]),
                     "+v"(av[4][0]), "+v"(av[4][1]), "+v"(av[5][0]), "+v"(av[5][1]),
                     "+v"(av[6][0]), "+v"(av[6][1]), "+v"(av[7][0]), "+v"(av[7][1]));
        asm volatile("" : "+v"(wd[0][0]), "+v"(wd[0][1]), "+v"(wd[1][0]), "+v"(wd[1][1]),
                     "+v"(wd[2][0]), "+v"(wd[2][1]), "+v"(wd[3][0]), "+v"(wd[3][1]),
                     "+v"(sbyte[0][0]), "+v"(sbyte[0][1]), "+v"(sbyte[1][0]), "+v"(sbyte[1][1]),
                     "+v"(sbyte[2][0]), "+v"(sbyte[2][1]), "+v"(sbyte[3][0]), "+v"(sbyte[3][1]));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          v8h bq[2][2];
#pragma unroll
          for (int nb2 = 0; nb2 < 2; ++nb2) {
            const v2h sb2 = e4m3_pair_f16(sbyte[kb][nb2]);
            bq[nb2][0] = decode_nv8_f16(wd[kb][nb2].x, sb2);
            bq[nb2][1] = decode_nv8_f16(wd[kb][nb2].y, sb2);
          }
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
            for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
              for (int nb2 = 0; nb2 < 2; ++nb2)
                acc2[mb2][nb2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    av[2 * kb + u2][mb2], bq[nb2][u2], acc2[mb2][nb2], 0, 0, 0);
        }
        continue;
      }
      // this wave's weight fragments and scales for the chunk
      uint4 wv[NGW][W8 ? 2 : 1];
      float sc[NGW][2];
#pragma unroll
      for (int q = 0; q < NGW; ++q) {
        const uint8_t* fp = st + OFF_B + (wave * NGW + q) * WFRAG + lane * 16;
        wv[q][0] = *reinterpret_cast<const uint4*>(fp);
        if (W8) wv[q][W8 ? 1 : 0] = *reinterpret_cast<const uint4*>(fp + 1024);
        if (WFMT == FP4MOE_W_MXFP4) {
          const uint32_t b = st[OFF_BS + (wave * 2 + q / RUN) * RS + (q % RUN) * 64 + lane];
          sc[q][0] = sc[q][1] = __uint_as_float(b << 23);   // the exponent field is the E8M0 byte
        } else if (WFMT == FP4MOE_W_NVFP4) {
          const uint32_t two = *reinterpret_cast<const uint16_t*>(
              st + OFF_BS + (wave * 2 + q / RUN) * RS + (q % RUN) * 128 + lane * 2);
          sc[q][0] = e4m3_to_f32(two & 0xffu);
          sc[q][1] = e4m3_to_f32(two >> 8);
        } else {
          sc[q][0] = sc[q][1] = 1.0f;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v8bf b[NGW];
#pragma unroll
        for (int q = 0; q < NGW; ++q) {
          if (WFMT == FP4MOE_W_MXFP4) {
            b[q] = decode_mx8(word(wv[q][0], t), sc[q][0]);
          } else if (WFMT == FP4MOE_W_NVFP4) {
            b[q] = decode_nv8(word(wv[q][0], t), sc[q][t >> 1]);
          } else {
            const uint4& h = wv[q][W8 ? (t >> 1) : 0];
            b[q] = decode_fp8x8(word(h, (t & 1) * 2), word(h, (t & 1) * 2 + 1));
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          v8bf a;
          if (AMX) {
            // own fragment slot (row mb*16 + l%16, block l/16), dword t
            const uint32_t d = *reinterpret_cast<const uint32_t*>(st + mb * 1024 + lane * 16 + t * 4);
            const uint32_t s8 = st[OFF_AS + (mb * 16 + r16) * 4 + g];
            a = decode_mx8(d, __uint_as_float(s8 << 23));
          } else {
            // fragment (mb, block l/16), slot (row l%16, K step t)
            a = as_bf8(*reinterpret_cast<const uint4*>(st + (mb * 4 + g) * 1024 + (r16 + 16 * t) * 16));
          }
#pragma unroll
          for (int q = 0; q < NGW; ++q)
            acc[mb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[q], acc[mb][q], 0, 0, 0);
        }
      }
    }
    wg_barrier();   // every wave is done with the ring before the next item refills it

    // epilogue: lane l holds rows 4*(l/16)+i of each M block, column l%16 of
    // each group
    float cs[NGW];
#pragma unroll
    for (int q = 0; q < NGW; ++q) {
      const int wrow = grp_run[q / RUN] * 16 + (q % RUN) * 16 + r16;
      if (WFMT == FP4MOE_W_NVFP4) cs[q] = p.w_tensor_scale[e];
      else if (WFMT == FP4MOE_W_FP8) cs[q] = p.w_channel_scale[(int64_t)e * p.N + wrow];
      else cs[q] = 1.0f;
    }
    if constexpr (AF16) {
      // 32x32 result layout: element i of lane l is row 8*(i/4) + 4*(l/32) +
      // i%4 of the M block, column l%32 of the two groups
      const float cs2 = p.w_tensor_scale[e] * *p.a_f16_scale;
      const int l32 = lane & 31, hh = lane >> 5;
      const int colw = nb * OUT_PER_WG + wave * OUT_PER_WAVE + l32;
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = tile_row0 + 32 * mb2 + 8 * (i / 4) + 4 * hh + (i % 4);
          if (r >= row_end) continue;
          if (STAGE == 1) {
            const float h = silu_mul(acc2[mb2][0][i] * cs2, acc2[mb2][1][i] * cs2);
            const int64_t o = (int64_t)r * p.ldo + colw;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          } else {
#pragma unroll
            for (int nb2 = 0; nb2 < 2; ++nb2) {
              const float y = acc2[mb2][nb2][i] * cs2;
              const int64_t o = (int64_t)r * p.ldo + colw + 32 * nb2;
              p.out[o] = (uint16_t)f32_to_bf16_rne(y);
              if (p.out_f32) p.out_f32[o] = y;
            }
          }
        }
      }
      continue;
    }
    const int col0 = nb * OUT_PER_WG + wave * OUT_PER_WAVE + r16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = tile_row0 + mb * 16 + g * 4 + i;
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < RUN; ++j) {
            const float h = silu_mul(acc[mb][j][i] * cs[j], acc[mb][j + RUN][i] * cs[j + RUN]);
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int q = 0; q < NGW; ++q) {
            const float y = acc[mb][q][i] * cs[q];
            const int64_t o = (int64_t)r * p.ldo + col0 + q * 16;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            if (p.out_f32) p.out_f32[o] = y;
          }
        }
      }
    }
  }
}

template <int WFMT, int AFMT, int STAGE, int NGW, int NW>
static void launch_dqt_stage(const GemmParams& p, int max_tiles, hipStream_t s) {
  // 32 groups per tile fit a 3-stage ring; 16 groups a 4-stage ring (3 with
  // FP8 fragments and bf16 activations)
  constexpr int S = (NGW * NW == 32 || (WFMT == FP4MOE_W_FP8 && AFMT == FP4MOE_A_BF16)) ? 3 : 4;
  const int out_per_wg = ((STAGE == 1) ? 8 : 16) * NGW * NW;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  const int cap = grid_cap() / 8;        // one workgroup per CU
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((dqt_gemm_kernel<WFMT, AFMT, STAGE, S, NGW, NW>), dim3(grid), dim3(64 * NW), 0,
                     s, p);
}

// FP4 weights with bf16 activations, when the output width allows: eight
// waves (two per SIMD, so one decodes while the other multiplies) of four
// groups, a tile 512 weight rows wide (half the activation copies per weight
// byte).  Otherwise four waves of four groups.
static bool wide_dqt(int wfmt, int afmt, int stage, int n_out) {
  return wfmt != FP4MOE_W_FP8 && afmt != FP4MOE_A_MXFP4 && n_out % (stage == 1 ? 256 : 512) == 0;
}

template <int WFMT, int AFMT>
static void launch_dqt_fmt(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  const int n_out = stage == 1 ? p.N / 2 : p.N;
  if constexpr (WFMT != FP4MOE_W_FP8 && AFMT != FP4MOE_A_MXFP4) {
    if (wide_dqt(WFMT, AFMT, stage, n_out)) {
      if (stage == 1) launch_dqt_stage<WFMT, AFMT, 1, 4, 8>(p, max_tiles, s);
      else launch_dqt_stage<WFMT, AFMT, 2, 4, 8>(p, max_tiles, s);
      return;
    }
  }
  if (stage == 1) launch_dqt_stage<WFMT, AFMT, 1, 4, 4>(p, max_tiles, s);
  else launch_dqt_stage<WFMT, AFMT, 2, 4, 4>(p, max_tiles, s);
}

bool dqt_supported(const GemmParams& p, int stage) {
  const int n_out = stage == 1 ? p.N / 2 : p.N;
  return p.block_m == 64 && p.w_layout == FP4MOE_LAYOUT_FRAGMENT &&
         n_out % (stage == 1 ? 128 : 256) == 0;
}

void launch_dqt_gemm(const GemmParams& p, int wfmt, int afmt, int stage, int max_tiles,
                     hipStream_t s) {
  if (afmt == FP4MOE_A_F16) {
    launch_dqt_fmt<FP4MOE_W_NVFP4, FP4MOE_A_F16>(p, stage, max_tiles, s);
  } else if (afmt == FP4MOE_A_BF16) {
    if (wfmt == FP4MOE_W_MXFP4) launch_dqt_fmt<FP4MOE_W_MXFP4, FP4MOE_A_BF16>(p, stage, max_tiles, s);
    else if (wfmt == FP4MOE_W_NVFP4) launch_dqt_fmt<FP4MOE_W_NVFP4, FP4MOE_A_BF16>(p, stage, max_tiles, s);
    else launch_dqt_fmt<FP4MOE_W_FP8, FP4MOE_A_BF16>(p, stage, max_tiles, s);
  } else {
    launch_dqt_fmt<FP4MOE_W_FP8, FP4MOE_A_MXFP4>(p, stage, max_tiles, s);
  }
}

}  // namespace fp4moe
