// fp4_grouped_gemm entry point: argument checks and family dispatch.  The
// kernels live in gemm_dq.hip / gemm_dqt.hip (bf16 or f16 MFMA on decoded
// weights), gemm_nvf16.hip (NVFP4 x f16 in 128-row tiles) and gemm_mx.hip
// (scaled FP4 / FP8 MFMA); gemm_common.h holds the operand conventions.
#include "gemm_common.h"

namespace fp4moe {

// NVFP4 weights x f16 activations, 128-row tiles (gemm_nvf16.hip): block_m
// 128, fragment weights, K a multiple of 512, output width a multiple of 128
// (stage 1) or 256 (stage 2); `queue` (optional) the work queue.
void launch_nvf16_gemm(const GemmParams& p, int stage, int max_tiles, int* queue, hipStream_t s);

// ===========================================================================
// dispatch
// ===========================================================================

// compute-unit count per device ordinal, read once (0 = not read yet); a
// racing first read stores the same value
static int g_num_cus[64] = {};

int grid_cap() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int n = (dev >= 0 && dev < 64) ? g_num_cus[dev] : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    if (dev >= 0 && dev < 64) g_num_cus[dev] = n;
  }
  return n * 8;
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int fp4_grouped_gemm(const fp4moe_gemm_args* a, void* stream) {
  FP4MOE_REQUIRE(a, "fp4_grouped_gemm: null args");
  FP4MOE_REQUIRE(a->stage == 1 || a->stage == 2, "fp4_grouped_gemm: stage=%d", a->stage);
  const bool mx = a->afmt == FP4MOE_A_MXFP4 && a->wfmt == FP4MOE_W_MXFP4;
  // FP8 weights x MXFP4 activations on the scaled MFMA: 192-row tiles
  const bool mx8 = a->afmt == FP4MOE_A_MXFP4 && a->wfmt == FP4MOE_W_FP8 && a->block_m == 192;
  // FP8 weights x FP8 activations (W8A8): 128-row tiles on the scaled MFMA
  const bool f8f8 = a->afmt == FP4MOE_A_FP8;
  const bool dq = !mx && !mx8 && !f8f8;
  FP4MOE_REQUIRE(a->afmt == FP4MOE_A_BF16 || a->afmt == FP4MOE_A_MXFP4 ||
                     a->afmt == FP4MOE_A_F16 || a->afmt == FP4MOE_A_FP8,
                 "fp4_grouped_gemm: afmt=%d", a->afmt);
  FP4MOE_REQUIRE(!f8f8 || (a->wfmt == FP4MOE_W_FP8 && a->block_m == 128 &&
                           a->w_layout == FP4MOE_LAYOUT_FRAGMENT &&
                           a->a_layout == FP4MOE_A_LAYOUT_CHUNKED),
                 "fp4_grouped_gemm: FP8 activations need FP8 fragment-major weights, block_m "
                 "128 and chunk-major activations");
  FP4MOE_REQUIRE(a->wfmt == FP4MOE_W_MXFP4 || a->wfmt == FP4MOE_W_NVFP4 || a->wfmt == FP4MOE_W_FP8,
                 "fp4_grouped_gemm: wfmt=%d", a->wfmt);
  FP4MOE_REQUIRE(!(a->wfmt == FP4MOE_W_NVFP4 && a->afmt == FP4MOE_A_MXFP4),
                 "fp4_grouped_gemm: NVFP4 weights take bf16 activations (nvfp4_qdq output)");
  // f16 activations: the NVFP4 tiled path only (E2M1 x E4M3 is exact in f16)
  const bool f16a = a->afmt == FP4MOE_A_F16;
  FP4MOE_REQUIRE(!f16a || (a->wfmt == FP4MOE_W_NVFP4 && (a->block_m == 64 || a->block_m == 128) &&
                           a->w_layout == FP4MOE_LAYOUT_FRAGMENT &&
                           a->a_layout == FP4MOE_A_LAYOUT_ROWMAJOR),
                 "fp4_grouped_gemm: f16 activations need NVFP4 fragment-major weights, block_m "
                 "64 or 128 and row-major A");
  FP4MOE_REQUIRE(!f16a || a->block_m != 128 || a->K % 512 == 0,
                 "fp4_grouped_gemm: f16 activations with block_m 128 need K a multiple of 512 "
                 "(K=%d)", a->K);
  FP4MOE_REQUIRE(((uintptr_t)a->work_queue & 3) == 0,
                 "fp4_grouped_gemm: work_queue must be 4-byte aligned");
  FP4MOE_REQUIRE(!f16a || (a->stage == 1 ? a->N / 2 : a->N) % (a->stage == 1 ? 128 : 256) == 0,
                 "fp4_grouped_gemm: f16 activations need an output width that is a multiple "
                 "of 128 (stage 1) or 256 (stage 2)");
  FP4MOE_REQUIRE(a->K > 0 && a->K % 128 == 0, "fp4_grouped_gemm: K=%d not a multiple of 128", a->K);
  FP4MOE_REQUIRE(a->N > 0 && a->N % 32 == 0 && (a->stage == 2 || a->N % 64 == 0),
                 "fp4_grouped_gemm: N=%d (stage %d)", a->N, a->stage);
  if (dq) {
    FP4MOE_REQUIRE(a->block_m == 16 || a->block_m == 32 || a->block_m == 64 ||
                       (f16a && a->block_m == 128),
                   "fp4_grouped_gemm: block_m=%d not in {16,32,64} for this format pair",
                   a->block_m);
  } else if (mx8 || f8f8) {
    FP4MOE_REQUIRE(a->w_layout == FP4MOE_LAYOUT_FRAGMENT,
                   "fp4_grouped_gemm: block_m %d needs fragment-major weights", a->block_m);
    const int n_out = a->stage == 1 ? a->N / 2 : a->N;
    const int out_per_wg = a->stage == 1 ? 128 : 256;
    FP4MOE_REQUIRE(n_out % out_per_wg == 0,
                   "fp4_grouped_gemm: output width %d not a multiple of %d", n_out, out_per_wg);
  } else {
    FP4MOE_REQUIRE(a->block_m == 32 || a->block_m == 64 || a->block_m == 128 ||
                       a->block_m == 192 || a->block_m == 256,
                   "fp4_grouped_gemm: block_m=%d not in {32,64,128,192,256} for MXFP4 x MXFP4",
                   a->block_m);
    FP4MOE_REQUIRE(a->block_m != 192 || a->w_layout == FP4MOE_LAYOUT_FRAGMENT,
                   "fp4_grouped_gemm: block_m 192 needs fragment-major weights");
    const bool big = a->block_m >= 128;
    const int out_per_wg = (a->stage == 1 ? 64 : 128) * (a->block_m == 192 ? 4 : big ? 2 : 1);
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
  FP4MOE_REQUIRE(a->a_layout == FP4MOE_A_LAYOUT_ROWMAJOR || a->a_layout == FP4MOE_A_LAYOUT_CHUNKED,
                 "fp4_grouped_gemm: a_layout=%d", a->a_layout);
  const bool a_chunked = a->a_layout == FP4MOE_A_LAYOUT_CHUNKED;
  FP4MOE_REQUIRE(!a_chunked || mx8 || f8f8 ||
                     (mx && a->w_layout == FP4MOE_LAYOUT_FRAGMENT &&
                      (a->block_m == 128 || a->block_m == 192 || a->block_m == 256)),
                 "fp4_grouped_gemm: chunked activations need MXFP4 activations, fragment "
                 "weights and block_m 128, 192 or 256 (FP8 weights: 192)");
  // (an empty batch, max_rows 0, may come with an empty activation slab)
  FP4MOE_REQUIRE(!a_chunked || (a->a_rows >= (a->max_rows > 0 ? 1 : 0) && a->a_rows <= (1 << 26) &&
                                (a->a_row_gather || a->a_rows >= a->max_rows)),
                 "fp4_grouped_gemm: a_rows=%d (max_rows=%d)", a->a_rows, a->max_rows);
  // the LDS-DMA tiles (MXFP4 x MXFP4, fragment weights, block_m >= 128) address
  // row-major A rows with 32-bit byte offsets
  FP4MOE_REQUIRE(!((mx || mx8) && a->w_layout == FP4MOE_LAYOUT_FRAGMENT && a->block_m >= 128 &&
                   !a_chunked) ||
                     (int64_t)a->max_rows * (a->lda / 2) <= (int64_t)0xffffffff,
                 "fp4_grouped_gemm: row-major A of %d rows x lda %lld exceeds 4 GiB for block_m %d",
                 a->max_rows, (long long)a->lda, a->block_m);
  const int n_out = a->stage == 1 ? a->N / 2 : a->N;
  FP4MOE_REQUIRE(a->ldo >= n_out, "fp4_grouped_gemm: ldo=%lld < %d", (long long)a->ldo, n_out);
  // the 192-row tiles store 16-byte pieces of output rows
  FP4MOE_REQUIRE((a->block_m != 192 && !f8f8) ||
                     (a->ldo % 8 == 0 && ((uintptr_t)a->out & 15) == 0),
                 "fp4_grouped_gemm: block_m %d needs ldo %% 8 == 0 and a 16-byte aligned out",
                 a->block_m);
  FP4MOE_REQUIRE(a_chunked || (a->lda >= a->K && a->lda % 32 == 0), "fp4_grouped_gemm: lda=%lld",
                 (long long)a->lda);
  // the FP8 activation slab is addressed with 32-bit offsets within a K chunk
  FP4MOE_REQUIRE(!f8f8 || (int64_t)a->a_rows * 128 <= (int64_t)0xffffffff,
                 "fp4_grouped_gemm: a_rows=%d too large for FP8 activations", a->a_rows);
  const bool quant_out = a->out_q != nullptr || a->out_q_scale != nullptr;
  FP4MOE_REQUIRE(!quant_out || (a->out_q && a->out_q_scale && a->stage == 1 && a->block_m == 192 &&
                                a->afmt == FP4MOE_A_MXFP4 && !a->out_f32 &&
                                (a->N / 2) % 128 == 0),
                 "fp4_grouped_gemm: out_q needs both buffers, stage 1, block_m 192, MXFP4 "
                 "activations, no out_f32 and an output width that is a multiple of 128");
  FP4MOE_REQUIRE(!quant_out || (a->out_q_rows >= a->max_rows && a->out_q_rows <= (1 << 26)),
                 "fp4_grouped_gemm: out_q_rows=%d (max_rows=%d)", a->out_q_rows, a->max_rows);
  FP4MOE_REQUIRE(!quant_out || ((uintptr_t)a->out_q & 3) == 0,
                 "fp4_grouped_gemm: out_q must be 4-byte aligned");
  if (a->max_tiles == 0 || a->max_rows == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(a->w && a->a && a->expert_offsets && a->tiles && a->n_tiles &&
                     (a->out || quant_out),
                 "fp4_grouped_gemm: null pointer");
  FP4MOE_REQUIRE(a->wfmt == FP4MOE_W_FP8 || a->w_scale, "fp4_grouped_gemm: w_scale is null");
  FP4MOE_REQUIRE(a->wfmt != FP4MOE_W_NVFP4 || a->w_tensor_scale,
                 "fp4_grouped_gemm: NVFP4 needs w_tensor_scale");
  FP4MOE_REQUIRE(a->wfmt != FP4MOE_W_FP8 || a->w_channel_scale,
                 "fp4_grouped_gemm: FP8 needs w_channel_scale");
  FP4MOE_REQUIRE(a->afmt != FP4MOE_A_MXFP4 || a->a_scale,
                 "fp4_grouped_gemm: MXFP4 activations need a_scale");
  FP4MOE_REQUIRE(!f16a || a->a_f16_scale, "fp4_grouped_gemm: f16 activations need a_f16_scale");
  FP4MOE_REQUIRE(!f8f8 || a->a_row_scale, "fp4_grouped_gemm: FP8 activations need a_row_scale");
  FP4MOE_REQUIRE(((uintptr_t)a->w & 15) == 0 && ((uintptr_t)a->a & 15) == 0,
                 "fp4_grouped_gemm: w and a must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();

  GemmParams p{};
  p.N = a->N;
  p.K = a->K;
  p.n_experts = a->n_experts;
  p.block_m = a->block_m;
  p.gather_div = a->gather_div;
  p.w_layout = a->w_layout;
  p.a_layout = a->a_layout;
  p.a_rows = a->a_rows;
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
  p.q_codes = a->out_q;
  p.q_scales = a->out_q_scale;
  p.q_rows = a->out_q_rows;
  p.a_f16_scale = a->a_f16_scale;
  p.a_row_scale = a->a_row_scale;
  hipStream_t s = as_stream(stream);
  const int mt = a->max_tiles;
  const int st = a->stage;
  if (mx) launch_mx_gemm(p, st, mt, s);
  else if (mx8) launch_mx_fp8_wide_gemm(p, st, mt, s);
  else if (f8f8) launch_fp8_fp8_wide_gemm(p, st, mt, s);
  else if (f16a && a->block_m == 128) launch_nvf16_gemm(p, st, mt, a->work_queue, s);
  else if (dqt_supported(p, st)) launch_dqt_gemm(p, a->wfmt, a->afmt, st, mt, s);
  else launch_dq_gemm(p, a->wfmt, a->afmt, st, mt, s);
  return check_launch("fp4_grouped_gemm");
}

extern "C" int mxfp4_linear(const uint8_t* a_codes, const uint8_t* a_scales, int M, int K,
                            int a_layout, int64_t a_stride, const uint8_t* w,
                            const uint8_t* w_scale, int N, uint16_t* out, int64_t ldo,
                            float* out_f32, void* stream) {
  FP4MOE_REQUIRE(M >= 0, "mxfp4_linear: M=%d", M);
  FP4MOE_REQUIRE(K > 0 && K % 128 == 0, "mxfp4_linear: K=%d not a multiple of 128", K);
  FP4MOE_REQUIRE(N > 0 && N % 512 == 0, "mxfp4_linear: N=%d not a multiple of 512", N);
  FP4MOE_REQUIRE(a_layout == FP4MOE_A_LAYOUT_ROWMAJOR || a_layout == FP4MOE_A_LAYOUT_CHUNKED,
                 "mxfp4_linear: a_layout=%d", a_layout);
  const bool chunked = a_layout == FP4MOE_A_LAYOUT_CHUNKED;
  FP4MOE_REQUIRE(chunked ? (a_stride >= M && a_stride <= (1 << 26))
                         : (a_stride >= K && a_stride % 32 == 0 &&
                            (int64_t)M * (a_stride / 2) <= (int64_t)0xffffffff),
                 "mxfp4_linear: a_stride=%lld (M=%d, K=%d, layout %d)", (long long)a_stride, M, K,
                 a_layout);
  FP4MOE_REQUIRE(ldo >= N && ldo % 8 == 0, "mxfp4_linear: ldo=%lld", (long long)ldo);
  if (M == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(a_codes && a_scales && w && w_scale && out, "mxfp4_linear: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)a_codes & 15) == 0 && ((uintptr_t)w & 15) == 0 &&
                     ((uintptr_t)out & 15) == 0,
                 "mxfp4_linear: a_codes, w and out must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  GemmParams p{};
  p.N = N;
  p.K = K;
  p.n_experts = 1;
  p.block_m = 192;
  p.gather_div = 1;
  p.w_layout = FP4MOE_LAYOUT_FRAGMENT;
  p.a_layout = a_layout;
  p.a_rows = chunked ? (int)a_stride : 0;
  p.lda = chunked ? K : a_stride;
  p.ldo = ldo;
  p.w = w;
  p.w_scale = w_scale;
  p.a = a_codes;
  p.a_scale = a_scales;
  p.out = out;
  p.out_f32 = out_f32;
  p.dense_rows = M;
  launch_mx_dense_gemm(p, as_stream(stream));
  return check_launch("mxfp4_linear");
}
