// fp4_grouped_gemm, NVFP4 weights x f16 activations in 128-row tiles.
//
// [NVFP4] "Serving NVFP4 models on AMD Instinct MI355", "Weight Dequantization
// and Activation QDQ" and "Memory Management": the packed E2M1 weights and
// their E4M3 per-16 scales are expanded inside the GEMM tile; no wider copy of
// the weights exists in memory.  The activations arrive QDQ'd, as f16 values
// with a power-of-two factor taken out, so every product (E2M1 x E4M3) x
// (E2M1 x E4M3) is exact in the f16 MFMA; the fp32 tensor scales are applied
// once, in the epilogue.
//
// Tile: 128 rows (four 32-row blocks; blocks wholly past the expert's last row
// are neither copied nor multiplied) by 256 weight rows.  Four waves, one per
// SIMD, each owning 64 weight rows (two pairs of 16-row groups; stage 1: the
// gate pair and the up pair of the same 32 output columns) for all 128 rows
// and the whole K.  A weight slice is streamed and decoded once per 128 rows
// of its expert.
//
// Operand paths.  A wave's weights are its own, so it streams its fragment
// pieces and E4M3 scale bytes straight into registers, R chunks ahead, with
// ordinary loads: no LDS traffic for them.  The activation chunk is shared by
// the four waves: it goes global -> registers -> LDS (two stages) and is read
// back as the MFMA operand.  Every load is visible to the compiler, which
// places the waits.
//
// K order inside a 128-wide chunk.  The 32x32x16 f16 MFMA takes, in lane l,
// eight K values of row (A) or column (B) l % 32, and lane half h = l / 32
// decides which eight.  Any assignment of K indices works as long as both
// operands use it: K step u (0..7) of half h takes elements 64h + 8u .. +7.
// For the weights that is dword u % 4 of fragment piece (l % 16) + 16 (2h +
// u / 4) of the lane's group -- two 16-byte loads per group and chunk -- and
// one E4M3 scale per two K steps.  The activation stage holds 256 bytes per
// row, its sixteen 16-byte slots XOR-swizzled by the row index, so that 16
// consecutive lanes always touch 16 different slots: the operand reads and the
// stores into LDS are bank-conflict free.
#include <type_traits>

#include "gemm_common.h"

namespace fp4moe {

namespace {

// f(integral_constant<int, I>) for I = B .. E-1: register arrays indexed by I
// stay in registers (their indices are constants before any loop unrolling).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int NV_BM = 128;                 // rows per tile
constexpr int NV_STAGE_BYTES = NV_BM * 256;  // one activation chunk: 128 rows x 128 f16
constexpr int NV_STAGES = 2;

// One chunk of a wave's weights: [pair][piece] 16-byte E2M1 pieces and the
// two E4M3 bytes of each piece.
struct NvChunk {
  uint4 q[2][2];
  uint32_t s[2][2];
};

template <int STAGE, int NW, int NMB>
__device__ __forceinline__ void nv_item(const GemmParams& p, uint8_t* smem, int e, int nb,
                                        int tile_row0, int row_end) {
  // weight chunks in flight per wave (the same bytes in flight per CU for
  // four or eight waves)
  constexpr int NV_R = NW == 4 ? 4 : 2;
  // activation chunks in flight in registers (ahead of the LDS stage)
  constexpr int AD = NMB <= 2 ? 2 : 1;
  constexpr int NA = 8 * NMB / NW;         // 16-byte activation pieces per lane and chunk
  constexpr int A_ROWS = 4 * NW;           // activation rows per round of the workgroup's lanes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5, r16 = lane & 15;
  const int nkc = p.K / 128;
  const int G = p.N / 16;

  // this lane's weight group in each pair, and its pieces r16 + 32 hh (+16)
  const uint8_t* wp[2];
  const uint8_t* sp[2];
  static_for<0, 2>([&](auto nb2) {
    int g0;
    if (STAGE == 1) g0 = (nb2 == 0 ? 0 : G / 2) + nb * 2 * NW + wave * 2;
    else g0 = nb * 4 * NW + wave * 4 + nb2 * 2;
    const int g = g0 + (l32 >> 4);
    wp[nb2] = p.w + ((int64_t)e * G + g) * nkc * 1024 + (r16 + 32 * hh) * 16;
    sp[nb2] = p.w_scale + ((int64_t)e * nkc * G + g) * 128 + (r16 + 32 * hh) * 2;
  });
  const int64_t s_chunk = (int64_t)G * 128;
  auto load_w = [&](NvChunk& wc, int c) {
    const int cc = c < nkc ? c : nkc - 1;   // past the end: a harmless reload
    static_for<0, 2>([&](auto nb2) {
      static_for<0, 2>([&](auto j) {
        wc.q[nb2][j] = *reinterpret_cast<const uint4*>(wp[nb2] + (int64_t)cc * 1024 + j * 256);
        wc.s[nb2][j] = *reinterpret_cast<const uint16_t*>(sp[nb2] + cc * s_chunk + j * 32);
      });
    });
  };

  // activation pieces of this lane: rows (tid / 16) + A_ROWS k, 16-byte slot tid % 16
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const uint8_t* a_ptr[NA];
  static_for<0, NA>([&](auto k) {
    const int r = tile_row0 + (tid >> 4) + A_ROWS * k;
    const int rr = r < row_end ? r : tile_row0;   // rows past the end repeat the first row
    const int64_t arow = p.gather ? (int64_t)(p.gather[rr] / p.gather_div) : (int64_t)rr;
    a_ptr[k] = A + arow * p.lda * 2 + (tid & 15) * 16;
  });
  const uint32_t a_st = (uint32_t)((tid >> 4) * 256 + (((tid & 15) ^ ((tid >> 4) & 15)) * 16));
  // (native vectors: a plain load and store each, no aggregate copies)
  auto load_a = [&](v4u (&ar)[NA], int c) {
    const int cc = c < nkc ? c : nkc - 1;
    static_for<0, NA>([&](auto k) {
      ar[k] = *reinterpret_cast<const v4u*>(a_ptr[k] + (int64_t)cc * 256);
    });
  };
  auto store_a = [&](const v4u (&ar)[NA], int stage) {
    static_for<0, NA>([&](auto k) {
      *reinterpret_cast<v4u*>(smem + stage * NV_STAGE_BYTES + a_st + k * A_ROWS * 256) = ar[k];
    });
  };

  v16f acc[NMB][2];
  static_for<0, NMB>([&](auto mb2) {
    static_for<0, 2>([&](auto nb2) { acc[mb2][nb2] = v16f{}; });
  });

  // operand read offsets: row 32 mb2 + l32, logical slot 8 hh + u
  const uint32_t a_rd = (uint32_t)(l32 * 256);
  const int a_sw = l32 & 15;
  auto compute = [&](const NvChunk& wc, int stage) {
    const uint8_t* st = smem + stage * NV_STAGE_BYTES + a_rd;
    static_for<0, 8>([&](auto u) {
      v8h a[NMB];
      static_for<0, NMB>([&](auto mb2) {
        a[mb2] = *reinterpret_cast<const v8h*>(st + mb2 * 32 * 256 + (((8 * hh + u) ^ a_sw) * 16));
      });
      v8h b[2];
      static_for<0, 2>([&](auto nb2) {
        const uint32_t sbyte = (wc.s[nb2][u >> 2] >> (8 * ((u & 3) >> 1))) & 0xffu;
        b[nb2] = decode_nv8_f16(word(wc.q[nb2][u >> 2], u & 3), e4m3_pair_f16(sbyte));
      });
      static_for<0, NMB>([&](auto mb2) {
        static_for<0, 2>([&](auto nb2) {
          acc[mb2][nb2] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb2], b[nb2], acc[mb2][nb2], 0, 0, 0);
        });
      });
    });
  };

  // prologue: weights of chunks 0..R-1, activation chunk 0 into stage 0,
  // chunks 1..AD into registers
  NvChunk wr[NV_R];
  static_for<0, NV_R>([&](auto i) { load_w(wr[i], i); });
  v4u ar[AD][NA];
  load_a(ar[0], 0);
  store_a(ar[0], 0);
  static_for<1, AD + 1>([&](auto i) { load_a(ar[i % AD], i); });

  // iteration c: (1) chunk c+1's activations into stage (c+1) % 2, (2) load
  // chunk c+1+AD's activations into the registers just freed, (3) multiply
  // chunk c, (4) load chunk c+R's weights into the registers chunk c used.
  // The barrier at the top makes stage c % 2 visible and stage (c+1) % 2 free.
  // K is a multiple of 512, so the loop runs whole groups of four chunks and
  // every register index is static.  Loads past the last chunk reload it, and
  // the store after the last chunk fills a stage nobody reads: both keep the
  // loop free of branches, so the loads stay where they are issued.
  for (int c0 = 0; c0 < nkc; c0 += 4) {
    static_for<0, 4>([&](auto j) {
      const int c = c0 + j;
      wait_lgkm0();
      wg_barrier();
      store_a(ar[(j + 1) % AD], (j + 1) & 1);
      load_a(ar[(j + 1) % AD], c + 1 + AD);
      compute(wr[j % NV_R], j & 1);
      load_w(wr[j % NV_R], c + NV_R);
    });
  }
  wait_lgkm0();
  wg_barrier();   // every wave is done with the stages before the next item refills them

  // epilogue: element i of lane l is row 8 (i / 4) + 4 hh + i % 4 of the
  // 32-row block, column l32 of the pair
  const float cs2 = p.w_tensor_scale[e] * *p.a_f16_scale;
#pragma unroll
  for (int mb2 = 0; mb2 < NMB; ++mb2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = tile_row0 + 32 * mb2 + 8 * (i / 4) + 4 * hh + (i % 4);
      if (r >= row_end) continue;
      if (STAGE == 1) {
        const int col = nb * 32 * NW + wave * 32 + l32;
        const float h = silu_mul(acc[mb2][0][i] * cs2, acc[mb2][1][i] * cs2);
        const int64_t o = (int64_t)r * p.ldo + col;
        p.out[o] = (uint16_t)f32_to_bf16_rne(h);
        if (p.out_f32) p.out_f32[o] = h;
      } else {
#pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2) {
          const int col = nb * 64 * NW + wave * 64 + nb2 * 32 + l32;
          const float y = acc[mb2][nb2][i] * cs2;
          const int64_t o = (int64_t)r * p.ldo + col;
          p.out[o] = (uint16_t)f32_to_bf16_rne(y);
          if (p.out_f32) p.out_f32[o] = y;
        }
      }
    }
  }
}

// Cost of a tile's items for the split of the work between XCDs: a workgroup
// spends about as much per item on streaming and decoding its weight slice
// as on one 32-row block of MFMAs, so live blocks plus one.
__device__ inline int nv_tile_cost(const GemmParams& p, int t) {
  const int e = p.tiles[2 * t], mt = p.tiles[2 * t + 1];
  int rows = p.offsets[e + 1] - p.offsets[e] - mt * NV_BM;
  rows = rows < NV_BM ? rows : NV_BM;
  return (rows + 31) / 32 + 1;
}

// The tile-list split point of XCD x (0..8): the first tile at which the
// running cost reaches x/8 of the total, moved back to the first tile of its
// expert (an expert's tiles share their weight slices under one L2).  Wave 0
// computes it; every lane returns it.
__device__ inline int nv_split(const GemmParams& p, int n_tiles, int x, int lane) {
  const int per_lane = (n_tiles + 63) / 64;
  const int t0 = min(n_tiles, lane * per_lane), t1 = min(n_tiles, t0 + per_lane);
  int sum = 0;
  for (int t = t0; t < t1; ++t) sum += nv_tile_cost(p, t);
  int incl = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int total = __shfl(incl, 63);
  int bt = n_tiles;
  if (x < 8) {
    const int64_t target = (int64_t)total * x / 8;
    int run = incl - sum;
    for (int t = t0; t < t1; ++t) {
      if (run >= target) { bt = t; break; }
      run += nv_tile_cost(p, t);
    }
  }
  for (int d = 32; d >= 1; d >>= 1) bt = min(bt, __shfl_xor(bt, d));
  return bt < n_tiles ? bt - p.tiles[2 * bt + 1] : n_tiles;
}

// Work items are (M tile, column block) pairs, in (column block, M tile)
// order inside an expert: the M tiles that share a weight slice, and the
// column blocks of a single-tile expert that share an activation tile, are
// neighbours and run side by side.  Each XCD (workgroups blockIdx % 8) takes
// a contiguous range of the list.  Without a queue the range is an equal
// share of the items and its workgroups take every slots-th item; with a
// queue the range is an equal share of the cost and its workgroups take the
// next item from the XCD's counter as they free up (item costs differ up to
// fivefold with the live-block count), and the last workgroup out returns
// every counter to zero.
template <int STAGE, int NW>
__global__ __launch_bounds__(64 * NW, 1) void nvf16_gemm_kernel(GemmParams p, int* queue) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NV_STAGES * NV_STAGE_BYTES];
  __shared__ int s_split[2];
  __shared__ int s_item;
  constexpr int OUT_PER_WG = (STAGE == 1 ? 32 : 64) * NW;
  const int n_out = STAGE == 1 ? p.N / 2 : p.N;
  const int n_nb = n_out / OUT_PER_WG;
  const int n_tiles = *p.n_tiles;
  const int tid = threadIdx.x;

  constexpr int NX = 8;
  const int xcd = blockIdx.x % NX, slot = blockIdx.x / NX;
  const int slots = ((int)gridDim.x - xcd + NX - 1) / NX;
  int64_t w_begin, w_end;
  if (queue) {
    if (tid < 64) {
      const int b0 = nv_split(p, n_tiles, xcd, tid);
      const int b1 = nv_split(p, n_tiles, xcd + 1, tid);
      if (tid == 0) s_split[0] = b0, s_split[1] = b1;
    }
    __syncthreads();
    // (wave-uniform: held in scalar registers)
    w_begin = (int64_t)__builtin_amdgcn_readfirstlane(s_split[0]) * n_nb;
    w_end = (int64_t)__builtin_amdgcn_readfirstlane(s_split[1]) * n_nb;
  } else {
    const int64_t n_work = (int64_t)n_tiles * n_nb;
    const int64_t per = (n_work + NX - 1) / NX;
    w_begin = (int64_t)xcd * per;
    w_end = min(n_work, w_begin + per);
  }

  for (int64_t k = slot;; k += slots) {
    int64_t wi = w_begin + k;
    if (queue) {
      __syncthreads();                      // every wave has read the previous item
      if (tid == 0) s_item = atomicAdd(queue + xcd, 1);
      __syncthreads();
      wi = w_begin + __builtin_amdgcn_readfirstlane(s_item);
    }
    if (wi >= w_end) break;
    const int any_tile = (int)(wi / n_nb);
    const int e = p.tiles[2 * any_tile];
    const int t0 = any_tile - p.tiles[2 * any_tile + 1];
    const int m_tiles = (p.offsets[e + 1] - p.offsets[e] + NV_BM - 1) / NV_BM;
    const int local = (int)(wi - (int64_t)t0 * n_nb);
    const int nb = local / m_tiles, mt = local - nb * m_tiles;
    const int tile_row0 = p.offsets[e] + mt * NV_BM;
    const int row_end = min(p.offsets[e + 1], tile_row0 + NV_BM);
    switch ((row_end - tile_row0 + 31) / 32) {
      case 1: nv_item<STAGE, NW, 1>(p, smem, e, nb, tile_row0, row_end); break;
      case 2: nv_item<STAGE, NW, 2>(p, smem, e, nb, tile_row0, row_end); break;
      case 3: nv_item<STAGE, NW, 3>(p, smem, e, nb, tile_row0, row_end); break;
      default: nv_item<STAGE, NW, 4>(p, smem, e, nb, tile_row0, row_end); break;
    }
  }
  // Every workgroup's last (empty) take precedes its arrival; the last to
  // arrive zeroes the counters for the next call on the queue.
  if (queue && tid == 0) {
    __threadfence();
    if (atomicAdd(queue + NX, 1) == (int)gridDim.x - 1) {
      __threadfence();
      for (int i = 0; i <= NX; ++i) atomicExch(queue + i, 0);
    }
  }
}

}  // namespace

template <int STAGE, int NW>
static void launch_nvf16_stage(const GemmParams& p, int max_tiles, int* queue, hipStream_t s) {
  const int n_out = STAGE == 1 ? p.N / 2 : p.N;
  const int64_t work = (int64_t)max_tiles * (n_out / ((STAGE == 1 ? 32 : 64) * NW));
  const int cap = grid_cap() / 8;        // one workgroup per CU
  int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  // With a queue the items are split between the eight XCD groups by cost,
  // so any group may own items however few there are: every group needs a
  // workgroup (the fixed share gives group x items only when x < work).
  if (queue && grid < 8) grid = 8;
  hipLaunchKernelGGL((nvf16_gemm_kernel<STAGE, NW>), dim3(grid), dim3(64 * NW), 0, s, p, queue);
}

// Eight waves (two per SIMD: a tile 512 weight rows wide, half the activation
// reads per weight of four waves) when the output width allows, else four.
void launch_nvf16_gemm(const GemmParams& p, int stage, int max_tiles, int* queue, hipStream_t s) {
  const int n_out = stage == 1 ? p.N / 2 : p.N;
  const bool eight = n_out % (stage == 1 ? 256 : 512) == 0;
  if (stage == 1) {
    if (eight) launch_nvf16_stage<1, 8>(p, max_tiles, queue, s);
    else launch_nvf16_stage<1, 4>(p, max_tiles, queue, s);
  } else {
    if (eight) launch_nvf16_stage<2, 8>(p, max_tiles, queue, s);
    else launch_nvf16_stage<2, 4>(p, max_tiles, queue, s);
  }
}

}  // namespace fp4moe
