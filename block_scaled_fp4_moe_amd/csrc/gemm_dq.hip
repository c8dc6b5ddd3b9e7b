// fp4_grouped_gemm, dq family: bf16 (or MXFP4-decoded) activations times
// MXFP4 / NVFP4 / FP8 weights decoded to bf16 in registers, bf16 MFMA.
#include "dq_item.h"

namespace fp4moe {

// ===========================================================================
// dq family: bf16 activations, FP4 weights decoded in registers
// ===========================================================================

// The work items (dq_item.h) of one stage, the workgroups looping over them.
// Register use is bounded so that WPE waves fit on a SIMD: the decode stream
// needs many loads in flight per compute unit.
template <int WFMT, int AFMT, int STAGE, int MB, int NG, int U, int WPE, int NW>
__global__ __launch_bounds__(64 * NW, WPE) void dq_gemm_kernel(GemmParams p) {
  __shared__ float red[NW - 1][MB * NG * 4][64];
  const int n_nb = ((STAGE == 1) ? p.N / 2 : p.N) / dq_out_cols<STAGE, NG>();
  const int64_t n_work = (int64_t)(*p.n_tiles) * n_nb;
  for (int64_t wi = blockIdx.x; wi < n_work; wi += gridDim.x)
    dq_item<WFMT, AFMT, STAGE, MB, NG, U, NW>(p, wi, red);
}

template <int WFMT, int AFMT, int STAGE, int MB, int NG, int U, int WPE, int NW = 4>
static void launch_dq_cfg(const GemmParams& p, int max_tiles, hipStream_t s) {
  const int out_cols = (STAGE == 1) ? (NG / 2) * 16 : NG * 16;
  const int n_nb = ((STAGE == 1) ? p.N / 2 : p.N) / out_cols;
  const int64_t work = (int64_t)max_tiles * n_nb;
  // Up to 32 workgroups per CU: each takes about one work item, so the
  // hardware dispatcher balances the items as workgroups finish (measured
  // faster than fewer workgroups looping over several items).
  const int cap = grid_cap() * 4;
  const int grid = (int)(work < cap ? (work < 1 ? 1 : work) : cap);
  hipLaunchKernelGGL((dq_gemm_kernel<WFMT, AFMT, STAGE, MB, NG, U, WPE, NW>), dim3(grid),
                     dim3(64 * NW), 0, s, p);
}

template <int WFMT, int AFMT, int STAGE>
static void launch_dq(const GemmParams& p, int max_tiles, hipStream_t s) {
  // Four weight groups per item where the output width allows it: the
  // activation fragment of a chunk then serves twice the weight bytes.
  const int n_out = (STAGE == 1) ? p.N / 2 : p.N;
  const bool ng4 = n_out % 64 == 0 && (STAGE == 2 || n_out % 32 == 0);
  // MXFP4 decode fits four waves per SIMD; NVFP4 / FP8 decode needs more
  // registers per chunk and runs three.
  constexpr int WPE16 = (WFMT == FP4MOE_W_MXFP4) ? 4 : 3;
  switch (p.block_m) {
    case 16:
      if (ng4) launch_dq_cfg<WFMT, AFMT, STAGE, 1, 4, 2, WPE16>(p, max_tiles, s);
      else launch_dq_cfg<WFMT, AFMT, STAGE, 1, 2, 4, 2>(p, max_tiles, s);
      break;
    case 32: launch_dq_cfg<WFMT, AFMT, STAGE, 2, 2, 2, 2>(p, max_tiles, s); break;
    default: launch_dq_cfg<WFMT, AFMT, STAGE, 4, 2, 1, 2>(p, max_tiles, s); break;
  }
}

template <int WFMT, int AFMT>
static void launch_dq_stage(const GemmParams& p, int stage, int max_tiles, hipStream_t s) {
  if (stage == 1) launch_dq<WFMT, AFMT, 1>(p, max_tiles, s);
  else launch_dq<WFMT, AFMT, 2>(p, max_tiles, s);
}

void launch_dq_gemm(const GemmParams& p, int wfmt, int afmt, int stage, int max_tiles,
                    hipStream_t s) {
  if (afmt == FP4MOE_A_BF16) {
    if (wfmt == FP4MOE_W_MXFP4) launch_dq_stage<FP4MOE_W_MXFP4, FP4MOE_A_BF16>(p, stage, max_tiles, s);
    else if (wfmt == FP4MOE_W_NVFP4) launch_dq_stage<FP4MOE_W_NVFP4, FP4MOE_A_BF16>(p, stage, max_tiles, s);
    else launch_dq_stage<FP4MOE_W_FP8, FP4MOE_A_BF16>(p, stage, max_tiles, s);
  } else {
    launch_dq_stage<FP4MOE_W_FP8, FP4MOE_A_MXFP4>(p, stage, max_tiles, s);
  }
}

}  // namespace fp4moe
