/*
 * fp4moe -- routed-expert MoE layer with block-scaled FP4 weights, for AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory, keeps no device state and never
 *     synchronizes: each call enqueues its kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and returns.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns FP4MOE_ERR_INVALID_ARG and launches nothing.
 *     fp4moe_last_error() then returns a thread-local message.
 *   - Data-dependent conditions found on the device (ids out of range, NaN
 *     scales, inexact conversions) are reported through caller-provided
 *     device counters and status arrays, never by faulting.
 *   - bf16 tensors are passed as uint16_t bit patterns; FP4 payloads, E8M0,
 *     E4M3 and FP8 codes as uint8_t.  All matrices are row-major.
 *   - FP4 payloads pack element 2i in the low nibble and 2i+1 in the high
 *     nibble of byte i.  E2M1 magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6},
 *     bit 3 is the sign.  An E8M0 byte c scales by 2^(c-127); 255 is NaN.
 *     FP8 is OCP E4M3FN (bias 7, max 448, 0x7F/0xFF NaN).
 *
 * Sources (web pages, cited by title and section):
 *   [ATOM]  "Serve Kimi-K2.5-MXFP4 on MI355X with ATOM"
 *   [NVFP4] "Serving NVFP4 models on AMD Instinct MI355 accelerators"
 *   [GAUDI] "Kimi-K2.7-Code on Gaudi 2"
 *   [K3]    "Kimi K3 on MI355X"
 */
#ifndef FP4MOE_H
#define FP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP4MOE_OK = 0,
  FP4MOE_ERR_INVALID_ARG = 1,  /* bad shape, null pointer, unsupported combination   */
  FP4MOE_ERR_UNSUPPORTED = 2,  /* device is not gfx950                                */
  FP4MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace size */
  FP4MOE_ERR_LAUNCH = 4        /* the HIP runtime reported an error at launch          */
};

/* Weight formats of fp4_grouped_gemm. */
enum {
  FP4MOE_W_MXFP4 = 0,  /* E2M1 codes [E,N,K/2] + E8M0 scales [E,N,K/32]                     */
  FP4MOE_W_NVFP4 = 1,  /* E2M1 codes [E,N,K/2] + E4M3 scales [E,N,K/16] + fp32 tensor scale [E] */
  FP4MOE_W_FP8 = 2     /* E4M3 codes [E,N,K] + fp32 per-row channel scale [E,N]              */
};

/* Weight layouts of fp4_grouped_gemm (see fp4_weight_preshuffle). */
enum {
  FP4MOE_LAYOUT_ROWMAJOR = 0,  /* codes [E,N,K/2] (FP8 [E,N,K]), scales [E,N,K/32|K/16]       */
  FP4MOE_LAYOUT_FRAGMENT = 1   /* fragment-major, produced by fp4_weight_preshuffle          */
};

/* Activation formats of fp4_grouped_gemm. */
enum {
  FP4MOE_A_BF16 = 0,   /* bf16 [rows, K]: weights are decoded to bf16 inside the GEMM tile  */
  FP4MOE_A_MXFP4 = 1,  /* E2M1 codes [rows, K/2] + E8M0 [rows, K/32]: gfx950 scaled MFMA    */
  FP4MOE_A_F16 = 2,    /* f16 [rows, K] times the power of two *a_f16_scale: the f16 form
                          that nvfp4_qdq writes; NVFP4 weights decoded to f16 in the tile  */
  FP4MOE_A_FP8 = 3     /* E4M3 codes, chunk-major [K/128, a_rows, 128], times one float
                          per row (a_row_scale): fp8_quant_per_token's output (W8A8)       */
};

/* Layouts of MXFP4 activations (see mxfp4_quant_1x32_chunked). */
enum {
  FP4MOE_A_LAYOUT_ROWMAJOR = 0,  /* codes [rows, lda/2], scales [rows, lda/32]              */
  FP4MOE_A_LAYOUT_CHUNKED = 1    /* codes [K/128][a_rows][64 B], scales [K/128][a_rows][4 B] */
};

/* Thread-local description of the last non-OK status returned on this thread. */
const char* fp4moe_last_error(void);

/* Checks that the current HIP device is gfx950.  Returns FP4MOE_OK or
 * FP4MOE_ERR_UNSUPPORTED.  Every other entry point performs the same check
 * once per device. */
int fp4moe_init(void);

/*
 * moe_route -- grouped sigmoid top-k routing with a correction bias.
 * [GAUDI] "What was built": the grouped top-k router with sigmoid scoring and
 * a correction bias; introduction: DeepSeek-V3-style tower, 384 routed experts.
 * Per token t (float32 decisions, identical to the oracle's reading):
 *   s_e   = float32(1/(1+exp(-logit)))  evaluated in float64, rounded once
 *   key_e = float32(s_e + bias_e)
 *   n_group > 1: groups of E/n_group contiguous experts, group score =
 *   float32(top1 key + top2 key); the topk_group best groups are kept (ties:
 *   lower group index).  Then the topk best keys among kept experts in
 *   descending order (ties: lower id) give topk_ids[t, 0..topk-1].
 *   topk_w[t,j] = s_j / sum(s_selected) (if renormalize) * routed_scale.
 * logits float32 [T,E], bias float32 [E] (NULL = zeros) -> topk_ids int32
 * [T,topk], topk_w float32 [T,topk].
 * Requires 1 <= E <= 1024, E % n_group == 0, E/n_group >= 2 when n_group > 1,
 * 1 <= topk_group <= n_group, 1 <= topk <= topk_group*E/n_group, topk <= 32.
 */
int moe_route(const float* logits, const float* bias, int T, int E, int n_group,
              int topk_group, int topk, int renormalize, float routed_scale,
              int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_permute -- stable sort of the T*k (token, slot) pairs by expert.
 * [NVFP4] "Memory Management": only dispatched experts are touched;
 * [GAUDI] "What it taught about Gaudi": cost follows the routing, empty expert
 * slots are skipped; [K3]: expert tiles carry padding.
 * k = topk + n_shared; pair p = t*k + j; slot j >= topk is shared expert
 * E + (j - topk).  Ids outside [0,E) are dropped (pair_pos = -1, counted in
 * n_dropped).  Kept pairs are sorted by expert, ascending p within an expert.
 * Outputs (device):
 *   expert_offsets int32 [E+n_shared+1]  exclusive prefix sum of the counts
 *   sorted_pairs   int32 [T*k]           pair at each sorted position, -1 past the end
 *   pair_pos       int32 [T*k]           sorted position of each pair, -1 if dropped
 *   tiles          int32 [max_tiles, 2]  (expert, m_tile) for every block_m rows
 *                                         of every non-empty expert, in expert order
 *   n_tiles        int32 [1]
 *   n_dropped      int32 [1]
 * max_tiles = moe_permute_max_tiles(...).  The workspace (device, size from
 * moe_permute_workspace, may be 0 bytes for small T) holds per-block counts.
 * Requires T >= 0, 1 <= topk <= 32, 0 <= n_shared <= 8, 1 <= E+n_shared <= 4096,
 * 1 <= block_m <= 1024.
 */
int moe_permute_max_tiles(int T, int topk, int E, int n_shared, int block_m);
size_t moe_permute_workspace(int T, int topk, int E, int n_shared, int block_m);
int moe_permute(const int32_t* topk_ids, int T, int topk, int E, int n_shared, int block_m,
                void* workspace, size_t workspace_bytes, int32_t* expert_offsets,
                int32_t* sorted_pairs, int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles,
                int32_t* n_dropped, void* stream);

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs and errors as moe_permute
 * without the workspace: the per-chunk histograms of large batches live in a
 * buffer the library owns, one per device, of
 * moe_permute_noalloc_max_workspace() bytes (4 MiB), held until the process
 * ends.  A batch whose moe_permute_workspace() exceeds that returns
 * FP4MOE_ERR_WORKSPACE before any launch (with E + n_shared = 385 the limit
 * is about 2.8 M pairs).  The call allocates nothing; the first call on a
 * device looks up the buffer's device address.  Every call on one device
 * shares that device's buffer, so calls that overlap on one device (on
 * different streams without ordering between them) race; calls ordered on
 * one stream do not.
 */
size_t moe_permute_noalloc_max_workspace(void);
int moe_permute_noalloc(const int32_t* topk_ids, int T, int topk, int E, int n_shared,
                        int block_m, int32_t* expert_offsets, int32_t* sorted_pairs,
                        int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles, int32_t* n_dropped,
                        void* stream);

/*
 * moe_route_permute -- moe_route followed by moe_permute in one launch, for
 * decode-sized batches: T*(topk+n_shared) <= 1024.  [GAUDI] "What was built"
 * (the router) and [NVFP4] "Memory Management" (the dispatch), as for the two
 * calls; the outputs are bit-identical to moe_route then moe_permute with the
 * same arguments (no workspace is needed at these sizes).  Larger batches,
 * and any argument either call rejects, return FP4MOE_ERR_INVALID_ARG.
 */
int moe_route_permute(const float* logits, const float* bias, int T, int E, int n_group,
                      int topk_group, int topk, int renormalize, float routed_scale,
                      int n_shared, int block_m, int32_t* topk_ids, float* topk_w,
                      int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                      int32_t* tiles, int32_t* n_tiles, int32_t* n_dropped, void* stream);

/*
 * mxfp4_quant_1x32 -- dynamic 1x32 MXFP4 quantization of bf16 rows.
 * [ATOM] "Stage B: Dynamic Activation Quantization": live bf16 activations
 * become FP4 payloads plus E8M0 scales, one per 32 values along K.
 * Per 32-block: e = floor(log2 amax) - 2 clamped to [-127,127] (amax = 0 gives
 * -127), scale byte e+127; code = E2M1 nearest to x/2^e, ties to even,
 * saturating at +-6, sign kept.
 * x bf16 with row stride ldx (elements); output row r reads input row
 * row_gather[r] when row_gather != NULL.  row_count (device, NULL = M) limits
 * the rows processed; rows at or past it are not written.
 * -> codes uint8 [M, K/2], scales uint8 [M, K/32].  K % 32 == 0; x and
 * codes 16-byte aligned, ldx % 8 == 0.
 */
int mxfp4_quant_1x32(const uint16_t* x, int M, int K, int64_t ldx, const int32_t* row_gather,
                     const int32_t* row_count, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mxfp4_quant_1x32_chunked -- the same quantization as mxfp4_quant_1x32, with
 * the output in the chunk-major layout FP4MOE_A_LAYOUT_CHUNKED that the
 * prefill GEMM copies as whole contiguous tiles.  Output row o of a slab of
 * out_rows rows:
 *   codes  byte (c*out_rows + o)*64 + (k%128)/2   for element k, c = k/128
 *   scales byte (c*out_rows + o)*4 + (k%128)/32
 * Input row r (r < M, and r < *row_count when row_count != NULL) goes to
 * output rows row_map[r*map_k + j], j < map_k, when row_map != NULL (stage 1
 * passes moe_permute's pair_pos and k, so each token is read once and its
 * codes land in expert order; entries outside [0, out_rows) are skipped),
 * else to output row r (out_rows >= M).  Rows no input maps to are not
 * written.  K % 128 == 0.  codes [K/128, out_rows, 64], scales
 * [K/128, out_rows, 4]; x and codes 16-byte aligned, ldx % 8 == 0.
 */
int mxfp4_quant_1x32_chunked(const uint16_t* x, int M, int K, int64_t ldx, const int32_t* row_map,
                             int map_k, int out_rows, const int32_t* row_count, uint8_t* codes,
                             uint8_t* scales, void* stream);

/*
 * fp8_quant_per_token -- dynamic per-token FP8 quantization of bf16 rows (the
 * W8A8 activations).  [GAUDI] "Exact MXFP4 to FP8 per-channel conversion":
 * the FP8 experts are served with dynamic per-token FP8 activations.
 * Per row r, IEEE float32 steps: s_r = amax_r / 448 (1 for an all-zero row);
 * code = E4M3FN of x / s_r, round to nearest even, saturating at +-448, the
 * sign of x kept (also for zero).
 * x bf16 [M, K] with row stride ldx (elements; ldx % 8 == 0); rows at or past
 * *row_count (device, NULL = M) are not written.  Output: codes chunk-major
 * [K/128, out_rows, 128] (row r's codes of K chunk c at (c*out_rows + r)*128)
 * and scales float [out_rows]; out_rows >= M.  K % 128 == 0, K <= 8192;
 * x and codes 16-byte aligned.
 */
int fp8_quant_per_token(const uint16_t* x, int M, int K, int64_t ldx, const int32_t* row_count,
                        int out_rows, uint8_t* codes, float* scales, void* stream);

/*
 * nvfp4_qdq -- NVFP4 quantize-dequantize round trip of bf16 activations.
 * [NVFP4] "Weight Dequantization and Activation QDQ".  IEEE float32 steps:
 *   s_t = tensor_scale_in ? *tensor_scale_in : amax(|x|)/2688 (1 if amax = 0)
 *   per 16-block: sb = E4M3_RNE_sat(amax_b / f32(6*s_t));
 *   code = E2M1_RNE_sat(x / f32(sb*s_t)) (all zero when sb = 0, sign kept);
 *   y = bf16(f32(q*sb) * s_t).
 * x, y bf16 [M,K] (K % 16 == 0); codes [M,K/2], scales_e4m3 [M,K/16] and
 * tensor_scale_out [1] are optional (NULL).  row_count as in mxfp4_quant_1x32.
 * y_f16 (optional, f16 [M,K]) receives y * 2^-p and y_f16_scale (optional,
 * [1]) receives 2^p, where 2^p <= s_t < 2^(p+1) (2^-126 for a zero or
 * subnormal s_t): the operand form of FP4MOE_A_F16.  For a positive finite
 * s_t every y * 2^-p is a multiple of 2^-17 below 5400 (|q*sb| lies in
 * [2^-10, 2688] and y has at most 8 significant bits), so y_f16 holds y
 * exactly.  y may be NULL when y_f16 is given.  The dynamic scale needs a workspace of
 * nvfp4_qdq_workspace() bytes.
 */
size_t nvfp4_qdq_workspace(void);
int nvfp4_qdq(const uint16_t* x, int M, int K, const int32_t* row_count,
              const float* tensor_scale_in, uint16_t* y, uint8_t* codes, uint8_t* scales_e4m3,
              float* tensor_scale_out, uint16_t* y_f16, float* y_f16_scale, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * fp4_grouped_gemm -- one GEMM stage over all expert segments.
 * [ATOM] "Stage D: MXFP4 Fused MoE" (stage 1 on fused gate/up weights, stage
 * 2 on down weights) and "When Is the Scale Applied?" (scale before the MFMA
 * for the bf16 path, inside the scaled MFMA for FP4 x FP4); [NVFP4] "Memory
 * Management" (MoE path: dequantization fused into the GEMM tile, no bf16
 * weight buffer); [GAUDI] "What was built" (gate and up rows concatenated).
 *   stage 1: per row r of expert e: [g | u] = A[r] . W_e^T (N = 2I, gate rows
 *            first); out[r, n] = bf16(SiLU(g_n) * u_n), n < I.
 *   stage 2: out[r, n] = bf16(A[r] . W_e^T), n < N.
 * Rows are the sorted pairs: expert e owns rows expert_offsets[e] ..
 * expert_offsets[e+1]-1; the tile list comes from moe_permute with the same
 * block_m.  A row r is read from A row a_row_gather[r] / gather_div when
 * a_row_gather != NULL (stage 1 passes sorted_pairs and k), else row r.
 * Supported (wfmt, afmt) and block_m:
 *   (MXFP4 | NVFP4 | FP8, BF16) and (FP8, MXFP4) with block_m in {16, 32, 64}:
 *     both operands decoded exactly to bf16 in registers, bf16 MFMA;
 *   (NVFP4, F16) with block_m 64 or 128 (see afmt FP4MOE_A_F16 below);
 *   (MXFP4, MXFP4) with block_m in {32, 64, 128, 192, 256}: the gfx950
 *     scaled MFMA, FP4 x FP4, both E8M0 scales as MFMA scale operands;
 *   (FP8, MXFP4) with block_m 192: the gfx950 scaled MFMA in its FP4 x FP8
 *     form (E4M3 weights, E2M1 activations, unit block scales), the per-row
 *     channel scale applied in the epilogue;
 *   (FP8, FP8) with block_m 128: W8A8 ([GAUDI] "Exact MXFP4 to FP8 per-channel
 *     conversion": per-channel FP8 weights, dynamic per-token FP8
 *     activations) on the gfx950 scaled MFMA with both operands E4M3 and unit
 *     block scales; a_row_scale[row] and the channel scale multiply the
 *     accumulators in the epilogue.  Fragment-major weights, a_layout
 *     FP4MOE_A_LAYOUT_CHUNKED (fp8_quant_per_token's layout; a row gather, if
 *     given, picks the activation row and its scale), no out_q.
 * K % 128 == 0, N % 32 == 0 (stage 1: N % 64 == 0).  The output width (N/2
 * in stage 1, N in stage 2) must be a multiple of: 64 / 128 for (MXFP4,
 * MXFP4) at block_m 32 or 64, 128 / 256 at block_m 128 or 256, 256 / 512 at
 * block_m 192; 128 / 256 for (FP8, MXFP4) at block_m 192, for (FP8, FP8) and
 * for (NVFP4, F16).  block_m 192 needs fragment-major weights.  With fragment-major
 * weights, block_m >= 128 and row-major A, the scaled-MFMA tiles need
 * max_rows * lda / 2 < 2^32 and gathered rows < max_rows.
 * a_layout FP4MOE_A_LAYOUT_CHUNKED (codes and scales of a_rows rows in the
 * layout of mxfp4_quant_1x32_chunked; lda unused) is taken by (MXFP4,
 * MXFP4) with fragment-major weights and block_m 128, 192 or 256, and by
 * (FP8, MXFP4) with block_m 192; other combinations return
 * FP4MOE_ERR_INVALID_ARG.  a_rows is in [1, 2^26] and at least max_rows
 * without a row gather; an empty batch (max_rows 0) may pass a_rows 0.
 * out_q / out_q_scale (stage 1, block_m 192, MXFP4 activations, out_f32 NULL):
 * the stage-1 output h is also written quantized exactly as
 * mxfp4_quant_1x32_chunked(bf16 h, out_rows = out_q_rows) writes it -- the
 * stage-2 activations of [ATOM] "Stage B" without a separate pass over h;
 * out may then be NULL (h not written in bf16).  Rows past a segment's end
 * are not written.
 * afmt FP4MOE_A_F16 (the f16 operand form of nvfp4_qdq; a_f16_scale points
 * to its power-of-two factor) is taken with NVFP4 fragment-major weights and
 * block_m 64 or 128 (128: K % 512 == 0): E2M1 times E4M3 is exact in f16 (at
 * most 6 significant bits, magnitudes 2^-10 .. 2688), so the products equal
 * those of the bf16 form and the factor is applied with the tensor scale in
 * the epilogue.
 */
typedef struct {
  int stage;               /* 1 or 2                                                */
  int wfmt;                /* FP4MOE_W_*                                            */
  int afmt;                /* FP4MOE_A_*                                            */
  int n_experts;           /* experts in the weight tensors (routed + shared)      */
  int N;                   /* weight rows per expert (stage 1: 2I)                 */
  int K;                   /* reduction length                                     */
  int max_rows;            /* rows of the sorted A / out buffers                   */
  int max_tiles;           /* rows of `tiles` (moe_permute_max_tiles)               */
  int block_m;             /* rows per tile                                        */
  int gather_div;          /* divisor applied to a_row_gather entries (>= 1)        */
  const uint8_t* w;        /* weight codes                                         */
  const uint8_t* w_scale;  /* E8M0 [E,N,K/32] | E4M3 [E,N,K/16] | unused (FP8)     */
  const float* w_tensor_scale;   /* NVFP4: [E]; else NULL                          */
  const float* w_channel_scale;  /* FP8: [E,N]; else NULL                          */
  const void* a;           /* bf16 [.,lda] or E2M1 codes [., lda/2]                */
  const uint8_t* a_scale;  /* MXFP4 activations: E8M0 [., K/32]                    */
  int64_t lda;             /* A row stride in ELEMENTS                             */
  const int32_t* a_row_gather;
  const int32_t* expert_offsets;
  const int32_t* tiles;
  const int32_t* n_tiles;
  uint16_t* out;           /* bf16 [max_rows, ldo]                                 */
  int64_t ldo;             /* out row stride in elements                           */
  float* out_f32;          /* optional float32 copy before bf16 rounding, stride ldo */
  int w_layout;            /* FP4MOE_LAYOUT_* of w and w_scale                      */
  int a_layout;            /* FP4MOE_A_LAYOUT_* of a and a_scale (MXFP4 only)       */
  int a_rows;              /* chunked layout: rows per K chunk slab of a / a_scale  */
  uint8_t* out_q;          /* optional: stage-1 output as MXFP4 codes, chunked      */
  uint8_t* out_q_scale;    /*   and its E8M0 scales (see below)                     */
  int out_q_rows;          /*   rows per K chunk slab of out_q / out_q_scale        */
  const float* a_f16_scale;  /* FP4MOE_A_F16: device [1], the power-of-two factor   */
  const float* a_row_scale;  /* FP4MOE_A_FP8: device [a_rows], one scale per row of a */
  int32_t* work_queue;     /* optional, (NVFP4, F16) at block_m 128: device int32 [16],
                              zero-filled once before its first use; every call leaves
                              it zero-filled.  Given, the workgroups take their items
                              from it as they free up (balanced by row count) instead
                              of a fixed share; calls sharing one queue must not
                              overlap (order them on one stream).  Other format pairs
                              ignore it.  NULL: the fixed share.                      */
} fp4moe_gemm_args;

int fp4_grouped_gemm(const fp4moe_gemm_args* args, void* stream);

/*
 * mxfp4_linear -- dense MXFP4 x MXFP4 linear layer: out = bf16(A . W^T).
 * [ATOM] "Stage C: MXFP4 Linear GEMM": activations quantized 1x32 on the fly
 * times a pre-shuffled MXFP4 weight on the gfx950 scaled MFMA -- the same
 * 192 x 512 tile as the prefill MoE GEMM, with one matrix and every row.
 *   A: M rows of MXFP4 activations; a_layout FP4MOE_A_LAYOUT_CHUNKED: the
 *      output of mxfp4_quant_1x32_chunked with out_rows = a_stride >= M;
 *      FP4MOE_A_LAYOUT_ROWMAJOR: codes [M, a_stride/2] + E8M0 [M, a_stride/32]
 *      (a_stride = row stride in elements, M * a_stride / 2 < 2^32).
 *   W: one [N, K] MXFP4 matrix in the fragment-major layout
 *      (fp4_weight_preshuffle with E = 1): codes and E8M0 scales.
 *   out: bf16 [M, ldo]; out_f32 (optional) the float32 values before rounding.
 * K % 128 == 0, N % 512 == 0, ldo % 8 == 0; a_codes, w and out 16-byte
 * aligned.  Device pointers owned by the caller; nothing is allocated.
 */
int mxfp4_linear(const uint8_t* a_codes, const uint8_t* a_scales, int M, int K, int a_layout,
                 int64_t a_stride, const uint8_t* w, const uint8_t* w_scale, int N, uint16_t* out,
                 int64_t ldo, float* out_f32, void* stream);

/*
 * fp4_weight_preshuffle -- rewrite static expert weights into the
 * fragment-major layout (FP4MOE_LAYOUT_FRAGMENT) that fp4_grouped_gemm
 * streams with one contiguous KiB per wavefront load.
 * [ATOM] "Stage C: MXFP4 Linear GEMM": the production FP4 GEMMs take their
 * weight operand pre-shuffled for the matrix instruction; this layout is our
 * own, derived from the MFMA operand layout of our kernels.
 * With G = N/16 row groups, C = K/128 chunks, f = (e*G + n/16)*C + k/128,
 * h = (e*C + k/128)*G + n/16 and lane = n%16 + 16*((k%128)/32), element
 * (e, n, k) goes to
 *   FP4 codes   byte f*1024 + lane*16 + (k%32)/2   (same nibble as before)
 *   FP8 codes   byte f*2048 + ((k%32)/16)*1024 + lane*16 + k%16
 *   E8M0 scale  byte h*64 + lane                     (MXFP4, per 32 along k)
 *   E4M3 scale  byte h*128 + lane*2 + (k%32)/16      (NVFP4, per 16 along k)
 * FP8 channel scales and NVFP4 tensor scales keep their layout.  Same sizes
 * as the inputs; out-of-place only.  codes [E,N,K/2] (FP8 [E,N,K]); scales
 * ignored (may be NULL) for FP8.  N % 16 == 0, K % 128 == 0.
 */
int fp4_weight_preshuffle(int wfmt, int E, int N, int K, const uint8_t* codes,
                          const uint8_t* scales, uint8_t* codes_out, uint8_t* scales_out,
                          void* stream);

/*
 * moe_combine -- weighted top-k combine.
 * [ATOM] "Stage D: MXFP4 Fused MoE" (stage-2 outputs reduced per token);
 * [K3]: the shared-expert contribution is added to the routed sum.
 * out[t] = bf16( sum_{j<topk} w[t,j] * y[pair_pos[t*k+j]]
 *              + sum_{i<n_shared} y[pair_pos[t*k+topk+i]] ), float32, j ascending;
 * pairs with pair_pos = -1 contribute nothing.  y bf16 [rows, H] (sorted
 * order); out bf16 [T,H]; out_f32 optional.  H % 8 == 0.
 */
int moe_combine(const uint16_t* y_sorted, const int32_t* pair_pos, const float* topk_w, int T,
                int topk, int n_shared, int H, uint16_t* out, float* out_f32, void* stream);

/*
 * moe_decode_fused -- the whole decode layer in one launch, for T <= 16
 * tokens: bf16 activations, MXFP4 weights in the fragment-major layout of
 * fp4_weight_preshuffle.
 * [GAUDI] "What was built" (decode kernels for at most 16 tokens that touch
 * only the routed experts); [ATOM] "Stage D: MXFP4 Fused MoE" (the
 * small-token down GEMM that reduces the experts' rows into the tokens
 * itself); [K3] "Copy inputs only for kernels that use them" (fixed
 * per-launch costs dominate small steps).
 * Computes exactly what moe_route_permute (block_m 16), fp4_grouped_gemm
 * stage 1 and stage 2 (MXFP4 x bf16, block_m 16) and moe_combine compute with
 * the same arguments, and writes the same outputs bit for bit: topk_ids
 * [T, topk], topk_w [T, topk], expert_offsets [E+n_shared+1], sorted_pairs
 * and pair_pos [T*k], tiles [max_tiles, 2] (max_tiles at least
 * moe_permute_max_tiles(T, topk, E, n_shared, 16)), n_tiles [1], n_dropped
 * [1], h bf16 [T*k, I] and y bf16 [T*k, H] in sorted order, out bf16 [T, H].
 * All experts are local (ids index the weight tensors directly).
 * Requires T <= 16, topk <= 16, n_shared <= 8, E + n_shared <= 1032, the
 * routing limits of moe_route, H and I multiples of 128; x, the weights, h,
 * y and out 16-byte aligned.
 * workspace: moe_decode_fused_workspace(H) bytes of device memory, zero-filled
 * by the caller before the first call; every completed call leaves it as a
 * later call needs it (word 0 and words 4.. back at zero, word 1 advanced).
 * Word 2 is a sticky flag the kernel sets if a wait at its grid barrier gave
 * up (never in a correct run; the outputs are then invalid); the caller
 * clears it.  The launch is cooperative (all workgroups resident at once) and
 * returns FP4MOE_ERR_LAUNCH if the device cannot host it.  Calls sharing one
 * workspace must not overlap.
 */
typedef struct {
  int T, H, I, E, n_shared, n_group, topk_group, topk, renormalize, max_tiles;
  float routed_scale;
  const uint16_t* x;        /* bf16 [T, H]                                     */
  const float* logits;      /* [T, E]                                          */
  const float* bias;        /* [E] or NULL                                     */
  const uint8_t* w13;       /* fragment-major MXFP4 [E+n_shared, 2I, H/2]      */
  const uint8_t* w13_scale; /* fragment-major E8M0 [E+n_shared, 2I, H/32]      */
  const uint8_t* w2;        /* fragment-major MXFP4 [E+n_shared, H, I/2]       */
  const uint8_t* w2_scale;  /* fragment-major E8M0 [E+n_shared, H, I/32]       */
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* sorted_pairs;
  int32_t* pair_pos;
  int32_t* tiles;
  int32_t* n_tiles;
  int32_t* n_dropped;
  uint16_t* h;
  uint16_t* y;
  uint16_t* out;
  void* workspace;
  size_t workspace_bytes;
} fp4moe_decode_args;
size_t moe_decode_fused_workspace(int H);
int moe_decode_fused(const fp4moe_decode_args* args, void* stream);

/*
 * mxfp4_to_fp8_channel -- exact MXFP4 -> FP8 E4M3 per-channel conversion.
 * [GAUDI] "Exact MXFP4 to FP8 per-channel conversion": per row, k = (exponent
 * of the row's largest element) - 7, each element becomes the E4M3 code of
 * x/2^k, channel_scale = 2^k.  Exact when the row's E8M0 scales span <= 9 binades.
 * row_status (optional): 0 exact, every element exponent in [-5,7];
 * 1 an element falls below the -5 floor; 2 a block has E8M0 255 (its codes
 * become 0x7F, k from the finite blocks); 3 the finite part of the row is
 * zero (k = 0).  n_inexact_rows (device, required) receives the number of
 * rows where some finite element is not reproduced exactly; the call sets it.
 * codes [rows, K/2], scales [rows, K/32] -> fp8 [rows, K], channel_scale
 * float32 [rows].  K % 32 == 0, K <= 32768; codes and fp8 16-byte aligned.
 */
int mxfp4_to_fp8_channel(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                         uint8_t* fp8, float* channel_scale, uint8_t* row_status,
                         uint32_t* n_inexact_rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4MOE_H */
