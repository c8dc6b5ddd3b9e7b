// fp4_grouped_gemm, mx family: MXFP4 activations times MXFP4 weights on the
// gfx950 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, E8M0 scale operands).
#include "gemm_common.h"

namespace fp4moe {

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
// WAVES_M x WAVES_N waves (4 in all); each wave owns WM M blocks x 8 weight
// groups of 16 rows (a 16*WM x 128 sub-tile, 32 MFMA tiles).  The
// workgroup tile is BM = 16*WM*WAVES_M rows by 128*WAVES_N weight rows.
//   WAVES_M = 2 (block_m 128): 128 x 256, two M tiles of an expert share a
//     weight slice through L2;
//   WAVES_M = 4 (block_m 256): 256 x 128, one workgroup covers every row of
//     a typical routed expert, so each weight byte is fetched from HBM once
//     whatever the timing of other workgroups; the activation chunk
//     (16 KiB) is what the workgroups of one XCD share through L2.
template <int STAGE, int WM, int WAVES_M, int WAVES_N, int S>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, WAVES_M * WAVES_N / 4) void mx_dma_gemm_kernel(GemmParams p) {
  constexpr int NW = WAVES_M * WAVES_N;             // waves per workgroup
  constexpr int BM = 16 * WM * WAVES_M;
  constexpr int WN = 8;                             // weight groups per wave
  constexpr int NG_WG = WN * WAVES_N;               // weight groups per workgroup
  constexpr int GPW = NG_WG / NW;                   // weight groups copied per wave
  constexpr int MBLK = BM / 16;                     // M blocks per tile
  constexpr int AMPW = MBLK / NW;                   // A blocks copied per wave
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (WN / 2) * 16 : WN * 16;
  constexpr int OUT_PER_WG = WAVES_N * OUT_PER_WAVE;
  constexpr int OFF_AS = BM * 64;                   // A codes: [MBLK][64 lanes][16 B]
  constexpr int OFF_B = OFF_AS + BM * 4;            // A scales: [row][4 blocks]
  constexpr int OFF_BS = OFF_B + NG_WG * 1024;      // B codes: [NG_WG groups][64 lanes][16 B]
  constexpr int STAGE_BYTES = OFF_BS + NW * 256;    // B scales: [NW waves][256 B]
  constexpr int D = AMPW + 1 + GPW + 1;             // DMA instructions per wave per chunk
  static_assert(D * (S - 2) <= 63, "vmcnt range");
  static_assert(S >= 3 && S <= 6, "ring depth");
  static_assert(S * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert(BM / 64 >= 1 && BM % 64 == 0 && NW >= BM / 64, "A scale copy: one dword per row");
  static_assert(GPW >= 1 && GPW <= 4 && AMPW >= 1, "copy split");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int g = lane >> 4, r16 = lane & 15;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int G = p.N / 16;
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  // row-major A: row stride lda/2 (scales lda/32), next chunk +64 (+4);
  // chunk-major A: row stride 64 (4), next chunk one slab of a_rows rows
  const bool chunked = p.a_layout == FP4MOE_A_LAYOUT_CHUNKED;
  const int64_t a_row_bytes = chunked ? 64 : p.lda / 2, a_srow = chunked ? 4 : p.lda / 32;
  const int64_t a_cstride = chunked ? (int64_t)p.a_rows * 64 : 64;
  const int64_t as_cstride = chunked ? (int64_t)p.a_rows * 4 : 4;
  const uint32_t smem_base = lds_offset(smem);

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  const int64_t per = (n_work + NX - 1) / NX;
  const int64_t w_begin = (int64_t)xcd * per;
  const int64_t w_end = min(n_work, w_begin + per);

  for (int64_t wi = w_begin + slot; wi < w_end; wi += slots) {
    // Items of one expert are ordered (column block, M tile): M tiles that
    // share a weight slice run side by side on one XCD.
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
    uint32_t a_off[AMPW];
#pragma unroll
    for (int j = 0; j < AMPW; ++j) {
      const int r = tile_row0 + (wave * AMPW + j) * 16 + r16;
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      a_off[j] = (uint32_t)(arow * a_row_bytes) + g * 16;
    }
    uint32_t as_off;
    {
      // BM/64 dword copies cover the tile's rows; with BM = 128 waves 2, 3
      // repeat the copies of waves 0, 1 (same bytes, same LDS slots)
      const int r = tile_row0 + (wave % (BM / 64)) * 64 + lane;
      int64_t arow = 0;
      if (r < row_end) arow = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
      as_off = (uint32_t)(arow * a_srow);
    }
    // The workgroup's NG_WG weight groups in LDS order: stage 1 gate groups
    // then the matching up groups.  Wave w copies LDS groups [w*GPW, +GPW),
    // one contiguous run of groups in the weight tensor.
    int grp0;
    {
      const int j0 = wave * GPW;
      if (STAGE == 1)
        grp0 = (j0 < NG_WG / 2) ? nb * (NG_WG / 2) + j0 : G / 2 + nb * (NG_WG / 2) + (j0 - NG_WG / 2);
      else
        grp0 = nb * NG_WG + j0;
    }
    const uint8_t* b_base = p.w + ((int64_t)e * G + grp0) * nkc * 1024;
    const uint32_t b_lane = lane * 16;
    // scales of the wave's GPW groups: GPW*64 bytes; lanes past that repeat
    const uint8_t* bs_base = p.w_scale + ((int64_t)e * nkc * G + grp0) * 64;
    const uint32_t bs_lane = (lane % (GPW * 16)) * 4;

    // copy chunk c into the ring stage of chunk slot q
    auto issue = [&](int c, int q) {
      const uint32_t st = smem_base + (uint32_t)((q % S) * STAGE_BYTES);
#pragma unroll
      for (int j = 0; j < AMPW; ++j)
        dma_b128(A + a_off[j] + (int64_t)c * a_cstride, st + (wave * AMPW + j) * 1024);
      dma_b32(p.a_scale + as_off + (int64_t)c * as_cstride, st + OFF_AS + (wave % (BM / 64)) * 256);
#pragma unroll
      for (int q = 0; q < GPW; ++q)
        dma_b128(b_base + ((int64_t)q * nkc + c) * 1024 + b_lane, st + OFF_B + (wave * GPW + q) * 1024);
      dma_b32(bs_base + (int64_t)c * G * 64 + bs_lane, st + OFF_BS + wave * 256);
    };

    // 32x32 output tiles: MT per wave in M, NT in N (32 weight rows each)
    constexpr int MT = WM / 2, NT = WN / 2;
    v16f acc[MT][NT];
#pragma unroll
    for (int mt2 = 0; mt2 < MT; ++mt2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt2][nt][i] = 0.f;

    // per-lane LDS read bases within a stage; fragments sit at constant offsets
    // The 32x32x64 MFMA takes, in lane l, row (or weight row) l % 32 and the
    // 32-element block l / 32 of a 64-wide K step.  In the ring both operands
    // sit as 16-row fragments (lane' = row % 16 + 16 * block of the 128-wide
    // chunk), so lane l of K step h reads fragment (l % 32) / 16 at lane'
    // l % 16 + 16 * (2h + l / 32): a per-lane base plus constant offsets.
    const int m16 = (lane & 31) >> 4, kb = lane >> 5;
    const int frag_lane = m16 * 1024 + (lane & 15) * 16 + kb * 256;
    const int a_lds = wm * WM * 1024 + frag_lane;
    const int as_lds = OFF_AS + wm * WM * 64 + (lane & 31) * 4 + kb;
    const int b_lds = OFF_B + frag_lane;
    const int bs_lds = OFF_BS + m16 * 64 + (lane & 15) + 16 * kb;

    // MFMA operands of one chunk (two 64-wide K steps), read from its ring
    // stage into registers
    v4u bo[2][NT], ao[2][MT];
    int bso[2][NT], aso[2][MT];
    auto read_ops = [&](int c) {
      const uint8_t* st = smem + (c % S) * STAGE_BYTES;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // first LDS group of the tile: stage 1 gate tiles then up tiles
          const int ju = (STAGE == 1)
                             ? ((nt < NT / 2) ? wn * (WN / 2) + nt * 2 : NG_WG / 2 + wn * (WN / 2) + (nt - NT / 2) * 2)
                             : wn * WN + nt * 2;
          bo[h][nt] = *reinterpret_cast<const v4u*>(st + b_lds + ju * 1024 + h * 512);
          bso[h][nt] = st[bs_lds + (ju / GPW) * 256 + (ju % GPW) * 64 + h * 32];
        }
#pragma unroll
        for (int mt2 = 0; mt2 < MT; ++mt2) {
          ao[h][mt2] = *reinterpret_cast<const v4u*>(st + a_lds + mt2 * 2048 + h * 512);
          aso[h][mt2] = st[as_lds + mt2 * 128 + 2 * h];
        }
      }
    };
    auto mma = [&]() {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt2 = 0; mt2 < MT; ++mt2) {
          const v8i af = v8i{(int)ao[h][mt2][0], (int)ao[h][mt2][1], (int)ao[h][mt2][2], (int)ao[h][mt2][3], 0, 0, 0, 0};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const v8i bf = v8i{(int)bo[h][nt][0], (int)bo[h][nt][1], (int)bo[h][nt][2], (int)bo[h][nt][3], 0, 0, 0, 0};
            acc[mt2][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[mt2][nt], 4, 4, 0,
                                                                           aso[h][mt2], 0, bso[h][nt]);
          }
        }
    };

    // Chunk c is multiplied from stage c % S while the copies of chunks
    // c+1 .. c+S-1 are in flight; the copy of chunk c+S-1 is issued right
    // after the barrier that retires chunk c-1's stage.
    for (int c = 0; c < S - 1 && c < nkc; ++c) issue(c, c);
    if constexpr (NW == 8) {
      // Ping-pong: the two waves of a SIMD (waves w and w+4) run half a
      // chunk apart, so one multiplies while the other reads its operands
      // from LDS.  All waves run the same loop; waves 4-7 start one barrier
      // late and waves 0-3 end with one extra barrier.  With barriers
      // numbered from 0, chunk c is read in half-step 2c by waves 0-3 and in
      // half-step 2c+1 by waves 4-7, and multiplied one half-step later.
      // Rules that keep the ring safe: every wave completes its LDS reads
      // before each barrier; chunk c has landed (every wave's copies) before
      // barrier 2c; the refill issued after a wave's first barrier of chunk
      // c targets chunk c-1's stage, last read before barrier 2c.
      const int grp = wave >> 2;
      if (grp == 1) {
        wait_chunks<D, S - 2>(min(S - 2, nkc - 1));
        wg_barrier();
      }
      // The barriers take the accumulators (first) and the operands (second)
      // as in/out register operands: the MFMAs of a chunk can then be moved
      // neither before the second barrier nor past the next first barrier,
      // which keeps each wave's multiply and read phases apart.
      static_assert(MT == 2 && NT == 4, "pinned barrier operand lists");
      for (int c = 0; c < nkc; ++c) {
        wait_chunks<D, S - 2>(min(S - 2, nkc - 1 - c));   // own copies of chunk c
        wait_lgkm0();
        asm volatile("s_barrier"
                     : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]),
                       "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3])
                     :
                     : "memory");
        if (c + S - 1 < nkc) issue(c + S - 1, c + S - 1);
        read_ops(c);
        // waves 4-7 pass barrier 2c+2 next: their copies of chunk c+1 must be in
        if (grp == 1 && c + 1 < nkc) wait_chunks<D, S - 2>(min(S - 2, nkc - 2 - c));
        wait_lgkm0();
        asm volatile("s_barrier"
                     : "+v"(bo[0][0]), "+v"(bo[0][1]), "+v"(bo[0][2]), "+v"(bo[0][3]),
                       "+v"(bo[1][0]), "+v"(bo[1][1]), "+v"(bo[1][2]), "+v"(bo[1][3]),
                       "+v"(ao[0][0]), "+v"(ao[0][1]), "+v"(ao[1][0]), "+v"(ao[1][1]),
                       "+v"(bso[0][0]), "+v"(bso[0][1]), "+v"(bso[0][2]), "+v"(bso[0][3]),
                       "+v"(bso[1][0]), "+v"(bso[1][1]), "+v"(bso[1][2]), "+v"(bso[1][3]),
                       "+v"(aso[0][0]), "+v"(aso[0][1]), "+v"(aso[1][0]), "+v"(aso[1][1])
                     :
                     : "memory");
        mma();
      }
      if (grp == 0) wg_barrier();
    } else {
      for (int c = 0; c < nkc; ++c) {
        wait_chunks<D, S - 2>(min(S - 2, nkc - 1 - c));
        wait_lgkm0();   // this wave's reads of chunk c-1 are complete: its stage is refilled next
        wg_barrier();
        if (c + S - 1 < nkc) issue(c + S - 1, c + S - 1);
        read_ops(c);
        mma();
      }
    }
    wg_barrier();   // every wave is done with the ring before the next item refills it

    // epilogue: lane l holds column l % 32 of each 32x32 tile and rows
    // (i / 4) * 8 + (l / 32) * 4 + i % 4 in accumulator element i
    const int col0 = nb * OUT_PER_WG + wn * OUT_PER_WAVE + (lane & 31);
    const int wrow0 = tile_row0 + wm * WM * 16 + kb * 4;
#pragma unroll
    for (int mt2 = 0; mt2 < MT; ++mt2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wrow0 + mt2 * 32 + (i >> 2) * 8 + (i & 3);
        if (r >= row_end) continue;
        if (STAGE == 1) {
#pragma unroll
          for (int j = 0; j < NT / 2; ++j) {
            const float h = silu_mul(acc[mt2][j][i], acc[mt2][j + NT / 2][i]);
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 32;
            p.out[o] = (uint16_t)f32_to_bf16_rne(h);
            if (p.out_f32) p.out_f32[o] = h;
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float y = acc[mt2][nt][i];
            const int64_t o = (int64_t)r * p.ldo + col0 + nt * 32;
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

// ---------------------------------------------------------------------------
// mx family, wide tiles (block_m 192): 192 rows x 512 weight rows (MXFP4
// weights) or x 256 weight rows (FP8 E4M3 weights with a per-row fp32 scale).
//
// At prefill sizes every weight byte comes from HBM once, while the
// activation rows of an expert are copied again for every column block of
// its weights.  A 192 x 512 tile needs half the activation copies of a
// 256 x 256 tile per weight byte, and 192 rows cover a uniformly routed
// expert (about T*k/E rows) with less padding.  The accumulators of the tile
// fill 3/4 of the register file: 8 waves (2 per SIMD) in a 2 (M) x 4 (N)
// grid, each wave 96 x 128 as 3 x 4 tiles of the 32x32x64 scaled MFMA, 192
// accumulator registers per lane.  That leaves room for the operands of one
// 64-wide K step only, so the ping-pong of the two waves of a SIMD runs at
// K-step granularity: per step a read phase (operands of one K step from
// LDS) and a multiply phase (12 MFMAs), one barrier each.
// Ring: 3 stages of one 128-wide K chunk (activation codes 12 KiB + scales
// 768 B, weight fragments 32 KiB + scales 2 KiB).  Every wave issues 7 DMA
// instructions per chunk: waves 0-3 two activation fragments, waves 4-7 one
// fragment and one 64-row scale copy (wave 7 repeats wave 6's scale copy:
// the same bytes to the same LDS addresses), then 4 weight fragments and
// their scales.
// W8: the weights are FP8 E4M3 fragments (16 rows x 128 K = 2 KiB, the two
// 16-value halves of every 32-value block 1 KiB apart) and enter the same
// scaled MFMA as format 0 (E2M1 activations stay format 4: the FP4 x FP8
// rate) with unit block scales; the per-row channel scale
// multiplies the accumulators in the epilogue.  The tile is 192 x 256 (4 x 64
// per wave in N, 3 x 2 MFMA tiles), so a stage holds activation codes and
// scales plus 32 KiB of weights; 6 DMA instructions per wave per chunk
// (4 for two 2 KiB weight fragments).
// LDS-DMA with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the saddr form): one VGPR per address instead of two.
__device__ __forceinline__ void dma_b128_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma_b32_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1"
               :: "v"(voff), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// A8 (with W8): W8A8, FP8 E4M3 activations with one float scale per row
// (fp8_quant_per_token, chunk-major) against the FP8 weight fragments, both
// MFMA format 0 with unit block scales; the row and channel scales multiply
// the accumulators in the epilogue.  A 16-row activation block of a chunk is
// laid out in LDS exactly like a weight fragment (2 KiB, the two 16-value
// halves of every 32-value block 1 KiB apart), so the two operands pair K
// the same way.  Tiles are 128 x 256 (a stage holds 16 KiB of activations
// and 32 KiB of weights; three 192-row stages would not fit the LDS), each
// wave 64 x 64 as 2 x 2 MFMA tiles; 6 DMA instructions per wave per chunk.
template <int STAGE, bool W8, bool A8 = false>
__global__ __launch_bounds__(512, 1) void mx_dma_wide_gemm_kernel(GemmParams p) {
  static_assert(!A8 || W8, "FP8 activations run against FP8 weights");
  constexpr int S = 3, NW = 8, BM = A8 ? 128 : 192;
  constexpr int WM = BM / 32, MT = BM / 64;         // 16-row blocks / 32-row tiles per wave
  constexpr int WN = W8 ? 4 : 8, NT = WN / 2;       // weight groups / 32-row tiles per wave
  constexpr int NG_WG = 4 * WN;                     // weight groups per workgroup
  constexpr int GPW = NG_WG / NW;                   // weight groups copied per wave
  constexpr int GB = W8 ? 2048 : 1024;              // bytes of one weight fragment
  constexpr int OUT_PER_WAVE = (STAGE == 1) ? (WN / 2) * 16 : WN * 16;
  constexpr int OUT_PER_WG = 4 * OUT_PER_WAVE;
  constexpr int OFF_AS = BM * (A8 ? 128 : 64);      // A codes: [blocks][64 lanes][16 B] (A8: [blocks][2 KiB])
  constexpr int OFF_B = OFF_AS + (A8 ? 0 : BM * 4); // A scales: [row][4 blocks] (none for A8)
  constexpr int OFF_BS = OFF_B + NG_WG * GB;        // B fragments: [NG_WG groups][GB]
  constexpr int STAGE_BYTES = OFF_BS + (W8 ? 0 : NW * 256);   // B scales: [8 waves][4 groups][64 B]
  constexpr int D = 2 + GPW * (GB / 1024) + (W8 ? 0 : 1);    // DMA instructions per wave per chunk
  constexpr int EP_TILES = (STAGE == 1) ? NT / 2 : NT;   // 32-column output tiles per wave
  constexpr int EP_COLS = 32 * EP_TILES;            // output columns per wave
  constexpr int EP_PITCH = EP_COLS * 2 + 64;        // epilogue LDS row: bf16 + bank skew
  static_assert(8 * 16 * EP_PITCH <= STAGE_BYTES, "epilogue buffers fit in one ring stage");
  static_assert(S * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert(OFF_B % 16 == 0 && OFF_BS % 16 == 0 && STAGE_BYTES % 16 == 0, "alignment");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                        // ping-pong group; also the M half
  const int wm = grp, wn = wave & 3;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int nkc = p.K / 128;
  const int G = p.N / 16;
  // dense mode (p.dense_rows > 0): one matrix, rows [0, dense_rows), the tile
  // list implicit
  const bool dense = p.dense_rows > 0;
  const int64_t n_tiles_all = dense ? (p.dense_rows + BM - 1) / BM : *p.n_tiles;
  const int64_t n_work = n_tiles_all * n_nb;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const bool chunked = p.a_layout == FP4MOE_A_LAYOUT_CHUNKED;
  const int64_t a_row_bytes = A8 ? 128 : (chunked ? 64 : p.lda / 2), a_srow = chunked ? 4 : p.lda / 32;
  const int64_t a_cstride = A8 ? (int64_t)p.a_rows * 128 : (chunked ? (int64_t)p.a_rows * 64 : 64);
  const int64_t as_cstride = chunked ? (int64_t)p.a_rows * 4 : 4;
  const uint32_t smem_base = lds_offset(smem);

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  const int64_t per = (n_work + NX - 1) / NX;
  const int64_t w_begin = (int64_t)xcd * per;
  const int64_t w_end = min(n_work, w_begin + per);

  // LDS read bases (see mx_dma_gemm_kernel): lane l of K step h reads
  // fragment (l % 32) / 16 at lane' l % 16 + 16 * (2h + l / 32)
  const int m16 = (lane & 31) >> 4, kb = lane >> 5;
  const int frag_lane = m16 * 1024 + (lane & 15) * 16 + kb * 256;
  const int a_lds = A8 ? (wm * WM + m16) * 2048 + (lane & 15) * 16 + kb * 1024
                      : wm * WM * 1024 + frag_lane;
  const int as_lds = OFF_AS + wm * WM * 64 + (lane & 31) * 4 + kb;
  // E4M3 operands of the 32x32x64 MFMA pair with E2M1 ones differently (read
  // on the device): with lane half kb of the E2M1 operand holding 32-value
  // block 2h+kb of K step h, lane half kb of the E4M3 operand holds 16-value
  // half kb of block 2h in its first 16 bytes and half kb of block 2h+1 in
  // its last 16 bytes.  In the fragment those halves sit at byte
  // kb*1024 + (row + 16*block)*16.
  const int b_lds = OFF_B + m16 * GB + (lane & 15) * 16 + (W8 ? kb * 1024 : kb * 256);
  const int bs_lds = OFF_BS + m16 * 64 + (lane & 15) + 16 * kb;

  for (int64_t wi = w_begin + slot; wi < w_end; wi += slots) {
    const int any_tile = (int)(wi / n_nb);
    const int e = dense ? 0 : p.tiles[2 * any_tile];
    const int t0 = dense ? 0 : any_tile - p.tiles[2 * any_tile + 1];
    const int seg0 = dense ? 0 : p.offsets[e], seg1 = dense ? p.dense_rows : p.offsets[e + 1];
    const int m_tiles = (seg1 - seg0 + BM - 1) / BM;
    const int local = (int)(wi - (int64_t)t0 * n_nb);
    const int nb = local / m_tiles, mt = local - nb * m_tiles;
    const int tile_row0 = seg0 + mt * BM;
    const int row_end = min(seg1, tile_row0 + BM);

    auto src_row = [&](int r) -> int64_t {
      if (r >= row_end) return 0;
      return p.gather ? (int64_t)(p.gather[r] / p.gather_div) : (int64_t)r;
    };
    // activation copies of this wave: fragments f0 (and f0+1 for waves 0-3),
    // waves 4-7 also one 64-row scale block; A8: both halves of 16-row block
    // `wave` (lane l: row l % 16, the 16-byte half of 32-value block l / 16)
    const int f0 = A8 ? wave : (grp == 0 ? 2 * wave : wave + 4);
    const uint32_t a_off0 = (uint32_t)(src_row(tile_row0 + f0 * 16 + r16) * a_row_bytes) + g * (A8 ? 32 : 16);
    const uint32_t a_off1 = (uint32_t)(src_row(tile_row0 + (f0 + 1) * 16 + r16) * a_row_bytes) + g * 16;
    const int sblk = grp == 0 ? 0 : min(wave - 4, 2);
    const uint32_t as_off = (uint32_t)(src_row(tile_row0 + sblk * 64 + lane) * a_srow);
    // weight groups [4w, 4w+4) of the workgroup: stage 1 gate groups then up groups
    int grp0;
    {
      const int j0 = wave * GPW;
      if (STAGE == 1)
        grp0 = (j0 < NG_WG / 2) ? nb * (NG_WG / 2) + j0 : G / 2 + nb * (NG_WG / 2) + (j0 - NG_WG / 2);
      else
        grp0 = nb * NG_WG + j0;
    }
    const uint8_t* b_base = p.w + ((int64_t)e * G + grp0) * nkc * GB;
    const uint8_t* bs_base = W8 ? nullptr : p.w_scale + ((int64_t)e * nkc * G + grp0) * 64;

    auto issue = [&](int c) {
      const uint32_t st = smem_base + (uint32_t)((c % S) * STAGE_BYTES);
      const uint8_t* a_c = A + (int64_t)c * a_cstride;
      if (A8) {
        dma_b128_s(a_c, a_off0, st + f0 * 2048);
        dma_b128_s(a_c, a_off0 + 16, st + f0 * 2048 + 1024);
      } else if (grp == 0) {
        dma_b128_s(a_c, a_off0, st + f0 * 1024);
        dma_b128_s(a_c, a_off1, st + (f0 + 1) * 1024);
      } else {
        dma_b128_s(a_c, a_off0, st + f0 * 1024);
        dma_b32_s(p.a_scale + (int64_t)c * as_cstride, as_off, st + OFF_AS + sblk * 256);
      }
#pragma unroll
      for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int hb = 0; hb < GB / 1024; ++hb)
          dma_b128_s(b_base + ((int64_t)q * nkc + c) * GB + hb * 1024, lane * 16,
                     st + OFF_B + (wave * GPW + q) * GB + hb * 1024);
      if (!W8) dma_b32_s(bs_base + (int64_t)c * G * 64, lane * 4, st + OFF_BS + wave * 256);
    };

    v16f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.f;

    // weight operand: FP4 one 16-byte piece (hi unused), FP8 the two halves;
    // activation operand likewise (ao_hi for A8 only)
    v4u bo[NT], bo_hi[NT], ao[MT], ao_hi[MT];
    int bso[NT], aso[MT];
    auto read_ops = [&](int c, int h) {
      const uint8_t* st = smem + (c % S) * STAGE_BYTES;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int ju = (STAGE == 1)
                           ? ((nt < NT / 2) ? wn * (WN / 2) + nt * 2 : NG_WG / 2 + wn * (WN / 2) + (nt - NT / 2) * 2)
                           : wn * WN + nt * 2;
        bo[nt] = *reinterpret_cast<const v4u*>(st + b_lds + ju * GB + h * 512);
        if (W8) {
          bo_hi[nt] = *reinterpret_cast<const v4u*>(st + b_lds + ju * GB + h * 512 + 256);
          bso[nt] = 127;
        } else {
          bso[nt] = st[bs_lds + (ju / GPW) * 256 + (ju % GPW) * 64 + h * 32];
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (A8) {
          ao[i] = *reinterpret_cast<const v4u*>(st + a_lds + i * 4096 + h * 512);
          ao_hi[i] = *reinterpret_cast<const v4u*>(st + a_lds + i * 4096 + h * 512 + 256);
          aso[i] = 127;
        } else {
          ao[i] = *reinterpret_cast<const v4u*>(st + a_lds + i * 2048 + h * 512);
          aso[i] = st[as_lds + i * 128 + 2 * h];
        }
      }
    };
    auto mma = [&]() {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const v8i af = A8 ? v8i{(int)ao[i][0], (int)ao[i][1], (int)ao[i][2], (int)ao[i][3],
                                (int)ao_hi[i][0], (int)ao_hi[i][1], (int)ao_hi[i][2], (int)ao_hi[i][3]}
                          : v8i{(int)ao[i][0], (int)ao[i][1], (int)ao[i][2], (int)ao[i][3], 0, 0, 0, 0};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (A8) {
            // A and B format 0 (E4M3), unit block scales
            const v8i bf = v8i{(int)bo[nt][0], (int)bo[nt][1], (int)bo[nt][2], (int)bo[nt][3],
                               (int)bo_hi[nt][0], (int)bo_hi[nt][1], (int)bo_hi[nt][2], (int)bo_hi[nt][3]};
            acc[i][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i][nt], 0, 0, 0,
                                                                        127, 0, 127);
          } else if (W8) {
            // A format 4 (E2M1), B format 0 (E4M3)
            const v8i bf = v8i{(int)bo[nt][0], (int)bo[nt][1], (int)bo[nt][2], (int)bo[nt][3],
                               (int)bo_hi[nt][0], (int)bo_hi[nt][1], (int)bo_hi[nt][2], (int)bo_hi[nt][3]};
            acc[i][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i][nt], 4, 0, 0,
                                                                        aso[i], 0, 127);
          } else {
            const v8i bf = v8i{(int)bo[nt][0], (int)bo[nt][1], (int)bo[nt][2], (int)bo[nt][3], 0, 0, 0, 0};
            acc[i][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i][nt], 4, 4, 0,
                                                                        aso[i], 0, bso[nt]);
          }
        }
      }
    };

    // Steps s = 2c + h.  Waves 0-3 pass barrier 2s before reading step s and
    // barrier 2s+1 before multiplying it; waves 4-7 run one barrier behind
    // (one extra barrier at the start, waves 0-3 one at the end).  Chunk c
    // has landed (every wave's copies) before barrier 4c: waves 0-3 wait
    // right before it, waves 4-7 before their second barrier of step 2c-1.
    // The refill of chunk c+2 goes into chunk c-1's stage, issued after
    // barrier 4c (4c+1 for waves 4-7); chunk c-1 was last read before 4c.
    for (int c = 0; c < S - 1 && c < nkc; ++c) issue(c);
    if (grp == 1) {
      wait_chunks<D, S - 2>(min(S - 2, nkc - 1));
      wg_barrier();
    }
    for (int c = 0; c < nkc; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0) wait_chunks<D, S - 2>(min(S - 2, nkc - 1 - c));
        wait_lgkm0();
        if constexpr (A8)
          asm volatile("s_barrier"
                       : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[MT - 1][0]), "+v"(acc[MT - 1][1])
                       :
                       : "memory");
        else if constexpr (W8)
          asm volatile("s_barrier"
                       : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),
                         "+v"(acc[MT - 1][0]), "+v"(acc[MT - 1][1])
                       :
                       : "memory");
        else
          asm volatile("s_barrier"
                       : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]),
                         "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3]),
                         "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[2][2]), "+v"(acc[2][3])
                       :
                       : "memory");
        if (h == 0 && c + S - 1 < nkc) issue(c + S - 1);
        read_ops(c, h);
        if (h == 1 && grp == 1 && c + 1 < nkc) wait_chunks<D, S - 2>(min(S - 2, nkc - 2 - c));
        wait_lgkm0();
        if constexpr (A8)
          asm volatile("s_barrier"
                       : "+v"(bo[0]), "+v"(bo[1]), "+v"(bo_hi[0]), "+v"(bo_hi[1]),
                         "+v"(ao[0]), "+v"(ao[MT - 1]), "+v"(ao_hi[0]), "+v"(ao_hi[MT - 1])
                       :
                       : "memory");
        else if constexpr (W8)
          asm volatile("s_barrier"
                       : "+v"(bo[0]), "+v"(bo[1]), "+v"(bo_hi[0]), "+v"(bo_hi[1]),
                         "+v"(ao[0]), "+v"(ao[1]), "+v"(ao[MT - 1]),
                         "+v"(aso[0]), "+v"(aso[1]), "+v"(aso[MT - 1])
                       :
                       : "memory");
        else
          asm volatile("s_barrier"
                       : "+v"(bo[0]), "+v"(bo[1]), "+v"(bo[2]), "+v"(bo[3]),
                         "+v"(ao[0]), "+v"(ao[1]), "+v"(ao[2]),
                         "+v"(bso[0]), "+v"(bso[1]), "+v"(bso[2]), "+v"(bso[3]),
                         "+v"(aso[0]), "+v"(aso[1]), "+v"(aso[2])
                       :
                       : "memory");
        mma();
      }
    }
    if (grp == 0) wg_barrier();
    wg_barrier();   // every wave is done with the ring before the next item refills it

    // epilogue: lane l holds column l % 32 of each 32x32 tile and rows
    // (i / 4) * 8 + (l / 32) * 4 + i % 4 in accumulator element i
    const int wrow0 = tile_row0 + wm * WM * 16;
    if constexpr (W8) {
      // per-row channel scales of the weight rows of this lane's columns
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int gbase = (STAGE == 1)
                              ? ((nt < NT / 2) ? nb * (NG_WG / 2) + wn * (WN / 2) + nt * 2
                                               : G / 2 + nb * (NG_WG / 2) + wn * (WN / 2) + (nt - NT / 2) * 2)
                              : nb * NG_WG + wn * WN + nt * 2;
        const float cs = p.w_channel_scale[(int64_t)e * p.N + gbase * 16 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int k = 0; k < 16; ++k) acc[i][nt][k] *= cs;
      }
    }
    if constexpr (A8) {
      // per-row activation scales (the row a sorted row reads)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int r = wrow0 + kb * 4 + i * 32 + (k >> 2) * 8 + (k & 3);
          const float sa = (r < row_end) ? p.a_row_scale[src_row(r)] : 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[i][nt][k] *= sa;
        }
    }
    if (p.out_f32) {
      // fp32 copy requested: element-wise stores of both outputs
      const int col0 = nb * OUT_PER_WG + wn * OUT_PER_WAVE + (lane & 31);
#pragma unroll
      for (int i3 = 0; i3 < MT; ++i3) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wrow0 + kb * 4 + i3 * 32 + (i >> 2) * 8 + (i & 3);
          if (r >= row_end) continue;
#pragma unroll
          for (int j = 0; j < EP_TILES; ++j) {
            const float y = (STAGE == 1) ? silu_mul(acc[i3][j][i], acc[i3][j + NT / 2][i]) : acc[i3][j][i];
            const int64_t o = (int64_t)r * p.ldo + col0 + j * 32;
            p.out[o] = (uint16_t)f32_to_bf16_rne(y);
            p.out_f32[o] = y;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // bf16 only: 16 rows at a time through this wave's slice of ring stage
      // 2 (the next item's prologue fills stages 0 and 1 only, and stage 2
      // after a barrier every wave passes once its epilogue is done), then
      // 16-byte row stores.  Lanes 2m and 2m+1 (columns 2m, 2m+1) swap one
      // value per row pair so that each writes one dword (two columns) of
      // one row: the even lane row i, the odd lane row i+1.
      uint8_t* ep = smem + 2 * STAGE_BYTES + wave * 16 * EP_PITCH;
      const bool odd = lane & 1;
      const int cpair = ((lane & 31) & ~1) * 2;     // byte offset of the column pair
      constexpr int LPR = EP_COLS * 2 / 16;         // lanes per 16-byte row piece set
      constexpr int RPI = 64 / LPR;                 // rows per 64-lane store
      const int64_t out_col = nb * OUT_PER_WG + wn * OUT_PER_WAVE + (lane % LPR) * 8;
#pragma unroll
      for (int i3 = 0; i3 < MT; ++i3) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < EP_TILES; ++j) {
#pragma unroll
            for (int i = 8 * hh; i < 8 * hh + 8; i += 2) {
              float v0, v1;
              if (STAGE == 1) {
                v0 = silu_mul(acc[i3][j][i], acc[i3][j + NT / 2][i]);
                v1 = silu_mul(acc[i3][j][i + 1], acc[i3][j + NT / 2][i + 1]);
              } else {
                v0 = acc[i3][j][i];
                v1 = acc[i3][j][i + 1];
              }
              const float send = odd ? v0 : v1;
              const float recv = __int_as_float(
                  __builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
              const float lo = odd ? recv : v0, hi = odd ? v1 : recv;
              const uint32_t packed = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
              const int row = (i >> 2) * 8 + kb * 4 + (i & 3) + (odd ? 1 : 0) - 16 * hh;
              *reinterpret_cast<uint32_t*>(ep + row * EP_PITCH + j * 64 + cpair) = packed;
            }
          }
#pragma unroll
          for (int q = 0; q < 16 / RPI; ++q) {
            const int row = q * RPI + lane / LPR;
            const uint4 v = *reinterpret_cast<const uint4*>(ep + row * EP_PITCH + (lane % LPR) * 16);
            const int r = wrow0 + i3 * 32 + hh * 16 + row;
            if (p.out && r < row_end) *reinterpret_cast<uint4*>(p.out + (int64_t)r * p.ldo + out_col) = v;
            if (STAGE == 1 && p.q_codes) {
              // MXFP4 of the bf16 row piece, as mxfp4_quant_1x32 computes it: a
              // 32-column block is 4 adjacent lanes (8 values each)
              const uint32_t w[4] = {v.x, v.y, v.z, v.w};
              uint32_t amax = 0;
#pragma unroll
              for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
              amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
              amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, false));
              const uint32_t sbyte = (uint32_t)max((int)(amax >> 7) - 2, 0);
              const float inv = __uint_as_float((254u - sbyte) << 23);   // 2^-e
              const uint32_t packed = e2m1_pack8(w, inv, amax > 0x7f80u);
              if (r < row_end) {
                const int64_t k = out_col;                  // h column of the lane's first value
                const int64_t slab = (k >> 7) * p.q_rows + r;
                *reinterpret_cast<uint32_t*>(p.q_codes + slab * 64 + ((k & 127) >> 1)) = packed;
                if ((lane & 3) == 0) p.q_scales[slab * 4 + ((k & 127) >> 5)] = (uint8_t)sbyte;
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

template <int STAGE, bool W8, bool A8 = false>
static void launch_mx_wide(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int out_per_wg = ((STAGE == 1) ? 256 : 512) / (W8 ? 2 : 1);
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  const int cap = grid_cap() / 8;        // one workgroup (eight waves) per CU
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((mx_dma_wide_gemm_kernel<STAGE, W8, A8>), dim3(grid), dim3(512), 0, s, p);
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

template <int STAGE, int WM, int WAVES_M, int WAVES_N, int S>
static void launch_mx_dma(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int out_per_wg = ((STAGE == 1) ? 64 : 128) * WAVES_N;
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / out_per_wg);
  int cap = grid_cap() / 8;              // one workgroup (four waves) per CU
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((mx_dma_gemm_kernel<STAGE, WM, WAVES_M, WAVES_N, S>), dim3(grid),
                     dim3(64 * WAVES_M * WAVES_N), 0, s, p);
}

template <int STAGE>
static void launch_mx(const GemmParams& p, int max_tiles, hipStream_t s) {
  const bool frag = p.w_layout == FP4MOE_LAYOUT_FRAGMENT;
  switch (p.block_m) {
    case 32: launch_mx_wm<STAGE, 1>(p, max_tiles, s); break;
    case 64: launch_mx_wm<STAGE, 2>(p, max_tiles, s); break;
    case 128:
      if (frag) launch_mx_dma<STAGE, 4, 2, 2, 4>(p, max_tiles, s);
      else launch_mx_lds<STAGE, 4>(p, max_tiles, s);
      break;
    case 192: launch_mx_wide<STAGE, false>(p, max_tiles, s); break;   // fragment weights only
    default:
      if (frag) launch_mx_dma<STAGE, 4, 4, 2, 4>(p, max_tiles, s);
      else launch_mx_lds<STAGE, 8>(p, max_tiles, s);
      break;
  }
}

void launch_mx_dense_gemm(const GemmParams& p, hipStream_t s) {
  launch_mx_wide<2, false>(p, (p.dense_rows + 191) / 192, s);
}

void launch_mx_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  if (stage == 1) launch_mx<1>(p, max_tiles, s);
  else launch_mx<2>(p, max_tiles, s);
}

void launch_mx_fp8_wide_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  if (stage == 1) launch_mx_wide<1, true>(p, max_tiles, s);
  else launch_mx_wide<2, true>(p, max_tiles, s);
}

void launch_fp8_fp8_wide_gemm(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  if (stage == 1) launch_mx_wide<1, true, true>(p, max_tiles, s);
  else launch_mx_wide<2, true, true>(p, max_tiles, s);
}

}  // namespace fp4moe
