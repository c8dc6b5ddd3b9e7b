// Dynamic activation quantization: mxfp4_quant_1x32, nvfp4_qdq and
// fp8_quant_per_token.
//
// mxfp4_quant_1x32 -- [ATOM] "Stage B: Dynamic Activation Quantization":
// bf16 activations become E2M1 payloads plus one E8M0 scale per 32 values.
// Scale rule (OCP MX): e = floor(log2 amax) - 2, clamped at -127.  For a bf16
// amax with biased exponent field f this is simply scale byte = max(f - 2, 0),
// so the scale is pure integer work on the bf16 bits.
//
// nvfp4_qdq -- [NVFP4] "Weight Dequantization and Activation QDQ":
// quantize-dequantize round trip before each GEMM; every step is an IEEE
// float32 operation with round-to-nearest-even.
//
// Layout: mxfp4_quant_1x32 gives each lane one whole 32-value block; in
// nvfp4_qdq each lane owns 8 consecutive bf16 (one 16-byte load), 2 lanes an
// NVFP4 block, with block maxima combined by xor shuffles.
#include "common.h"

namespace fp4moe {

__device__ __forceinline__ float e2m1_mag_value(uint32_t c) {
  // codes 0..7 -> 0, .5, 1, 1.5, 2, 3, 4, 6
  return c < 4 ? 0.5f * (float)c : (c == 7 ? 6.0f : (float)(c - 2));
}

// floor(log2 v) for a positive normal float.
__device__ __forceinline__ int floor_log2_f32(float v) {
  return (int)((__float_as_uint(v) >> 23) & 0xffu) - 127;
}

// Round a non-negative finite float to the nearest E4M3FN value (ties to
// even, saturating at 448).  Returns the value; *code receives the byte.
__device__ __forceinline__ float e4m3_rne_sat(float v, uint32_t* code) {
  if (!(v > 0.f)) {
    *code = 0;
    return 0.f;
  }
  if (v >= 448.f) {
    *code = 0x7e;
    return 448.f;
  }
  int e = (__float_as_uint(v) >> 23) == 0 ? -127 : floor_log2_f32(v);
  e = max(e, -6);
  const int qe = e - 3;                       // quantum 2^(e-3): 3 mantissa bits
  float r = rintf(v * exp2i(-qe)) * exp2i(qe);  // both scalings are exact
  r = fminf(r, 448.f);
  if (r == 0.f) {
    *code = 0;
  } else if (r >= 0.015625f) {
    const int E = floor_log2_f32(r);
    const uint32_t mant = (uint32_t)((r * exp2i(-E) - 1.f) * 8.f);
    *code = ((uint32_t)(E + 7) << 3) | mant;
  } else {
    *code = (uint32_t)(r * 512.f);            // subnormal: r = m * 2^-9
  }
  return r;
}

// ---- fp8_quant_per_token ------------------------------------------------
//
// [GAUDI] "Exact MXFP4 to FP8 per-channel conversion": the FP8 experts run
// with dynamic per-token FP8 activations.  Per row: s = amax / 448 (1 for a
// zero row) and code = E4M3(x / s), both IEEE float32 steps, the E4M3
// rounding to nearest even and saturating (e4m3_rne_sat).  One wavefront per
// row; lane l owns the 16-byte pieces l, l+64, ... of the row, held in
// registers between the maximum and the encode.  Output chunk-major: the 128
// codes of K chunk c of row r at (c * out_rows + r) * 128, so the GEMM copies
// a tile's chunk as 16-byte pieces of whole rows.
constexpr int kFp8MaxSteps = 16;   // K <= 64 lanes * 16 steps * 8 values = 8192

// STEPS: 16-byte pieces per lane held in registers, the smallest of 4 / 8 / 16
// that covers the row (fewer registers, more waves in flight for short rows).
template <int STEPS>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ x, int M,
                                                        int K, int64_t ldx,
                                                        const int32_t* __restrict__ row_count,
                                                        int out_rows, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = row_count ? min(M, *row_count) : M;
  if (r >= rows) return;
  const int pieces = K / 8;
  uint4 v[STEPS];
  float amax = 0.f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int j = lane + 64 * st;
    v[st] = make_uint4(0, 0, 0, 0);
    if (j < pieces) v[st] = *reinterpret_cast<const uint4*>(x + r * ldx + j * 8);
    const uint32_t w[4] = {v[st].x, v[st].y, v[st].z, v[st].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(w[i] & 0xffffu)), fabsf(bf16_to_f32(w[i] >> 16))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  if (lane == 0) scales[r] = sc;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int j = lane + 64 * st;
    if (j >= pieces) break;
    const uint32_t w[4] = {v[st].x, v[st].y, v[st].z, v[st].w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
      const float q = __fdiv_rn(bf16_to_f32(b), sc);
      uint32_t c;
      e4m3_rne_sat(fabsf(q), &c);
      c |= (b & 0x8000u) ? 0x80u : 0u;          // the sign of x (and of q), zero included
      out[i >> 2] |= c << (8 * (i & 3));
    }
    const int64_t chunk = j >> 4;
    *reinterpret_cast<uint2*>(codes + (chunk * out_rows + r) * 128 + (j & 15) * 8) =
        make_uint2(out[0], out[1]);
  }
}

// ---- mxfp4_quant_1x32 ---------------------------------------------------

// One lane per 32-value block: four 16-byte loads, the block maximum without
// cross-lane traffic, one 16-byte code store and one scale byte per output
// row.
// CHUNKED: output in the chunk-major layout, byte (c*out_rows + o)*64 +
// (k%128)/2 for codes and (c*out_rows + o)*4 + (k%128)/32 for scales
// (c = k/128), with output rows o = row_map[row*map_k + j] (entries outside
// [0, out_rows) skipped) or o = row without a map; else row-major [M, K/2]
// and [M, K/32], input row gather[row] when gather != NULL.
template <bool CHUNKED>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ row_map, int map_k, int out_rows,
    const int32_t* __restrict__ row_count, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int bpr = K / 32;                           // blocks per row
  const int rows = row_count ? min(M, *row_count) : M;
  const int64_t total = (int64_t)rows * bpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t row = t / bpr;
    const int b = (int)(t - row * bpr);
    const int64_t src = gather ? (int64_t)gather[row] : row;
    const uint4* xp = reinterpret_cast<const uint4*>(x + src * ldx + (int64_t)b * 32);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xp[q];
      w[4 * q] = v.x;
      w[4 * q + 1] = v.y;
      w[4 * q + 2] = v.z;
      w[4 * q + 3] = v.w;
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      amax = max(amax, w[i] & 0x7fffu);
      amax = max(amax, (w[i] >> 16) & 0x7fffu);
    }
    const int f = (int)(amax >> 7);                 // bf16 biased exponent of amax
    const uint32_t sbyte = (uint32_t)max(f - 2, 0);
    const float inv = __uint_as_float((254u - sbyte) << 23);   // 2^(127 - sbyte) = 2^-e
    const bool has_nan = amax > 0x7f80u;
    uint32_t packed[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) packed[d] = e2m1_pack8(w + 4 * d, inv, has_nan);
    const uint4 cv = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (CHUNKED) {
      const int n_dst = row_map ? map_k : 1;
      for (int j = 0; j < n_dst; ++j) {
        const int64_t o = row_map ? (int64_t)row_map[row * map_k + j] : row;
        if (o < 0 || o >= out_rows) continue;
        const int64_t slab = (int64_t)(b >> 2) * out_rows + o;
        *reinterpret_cast<uint4*>(codes + slab * 64 + (b & 3) * 16) = cv;
        scales[slab * 4 + (b & 3)] = (uint8_t)sbyte;
      }
    } else {
      *reinterpret_cast<uint4*>(codes + row * (K / 2) + (int64_t)b * 16) = cv;
      scales[row * bpr + b] = (uint8_t)sbyte;
    }
  }
}

// ---- nvfp4_qdq ----------------------------------------------------------

__global__ void nvfp4_zero_kernel(uint32_t* ws) { ws[0] = 0u; }

// Tensor amax: four independent 16-byte loads in flight per lane per step,
// one maximum per workgroup (LDS), one atomic per workgroup.
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const uint16_t* __restrict__ x, int M,
                                                         int K, const int32_t* __restrict__ row_count,
                                                         uint32_t* __restrict__ ws) {
  __shared__ uint32_t wave_max[4];
  const int rows = row_count ? min(M, *row_count) : M;
  const int64_t total = (int64_t)rows * (K / 8);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t amax = 0;
  for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < total; c0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + u * stride;
      v[u] = c < total ? xv[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        amax = max(amax, w[i] & 0x7fffu);
        amax = max(amax, (w[i] >> 16) & 0x7fffu);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    if (m) atomicMax(ws, m);
  }
}

__global__ __launch_bounds__(256) void nvfp4_qdq_kernel(
    const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ row_count,
    const float* __restrict__ ts_in, const uint32_t* __restrict__ ws, uint16_t* __restrict__ y,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ ts_out,
    uint16_t* __restrict__ y16, float* __restrict__ y16_scale) {
  float s_t;
  if (ts_in) {
    s_t = *ts_in;
  } else {
    const float amax_t = bf16_to_f32(*ws);
    s_t = amax_t > 0.f ? __fdiv_rn(amax_t, 2688.f) : 1.f;
  }
  if (ts_out && blockIdx.x == 0 && threadIdx.x == 0) *ts_out = s_t;
  // f16 operand form: y * 2^-p with 2^p the power of two at or below s_t
  uint32_t pbits = __float_as_uint(s_t) & 0x7f800000u;
  if (pbits == 0) pbits = 0x00800000u;
  const float p2 = __uint_as_float(pbits);
  const float inv_p2 = __fdiv_rn(1.f, p2);                   // exact: a power of two
  if (y16_scale && blockIdx.x == 0 && threadIdx.x == 0) *y16_scale = p2;
  const float denom = __fmul_rn(6.f, s_t);
  const int rows = row_count ? min(M, *row_count) : M;
  const int64_t total = (int64_t)rows * (K / 8);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c - threadIdx.x % 2 < total;
       c += stride) {
    const bool active = c < total;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (active) v = reinterpret_cast<const uint4*>(x)[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = max(amax, w[i] & 0x7fffu);
      amax = max(amax, (w[i] >> 16) & 0x7fffu);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
    uint32_t scode;
    const float sb = e4m3_rne_sat(__fdiv_rn(bf16_to_f32(amax), denom), &scode);
    const float d = __fmul_rn(sb, s_t);
    uint32_t packed = 0;
    uint32_t yo[4] = {0, 0, 0, 0};
    uint32_t ho[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const uint32_t sign = (h >> 15) & 1u;
      uint32_t mag = 0;
      uint32_t ybits = sign << 15;
      if (sb > 0.f) {
        const float q = __fdiv_rn(bf16_to_f32(h), d);
        mag = e2m1_mag_code(fabsf(q));
        const float qv = __fmul_rn(e2m1_mag_value(mag), sb);   // exact
        const float yv = __fmul_rn(sign ? -qv : qv, s_t);
        ybits = f32_to_bf16_rne(yv);
        if (mag == 0) ybits = sign << 15;
      }
      packed |= (mag | (sign << 3)) << (4 * i);
      yo[i >> 1] |= ybits << (16 * (i & 1));
      const _Float16 hv = (_Float16)(bf16_to_f32(ybits) * inv_p2);   // exact (see header)
      const uint32_t hb = __builtin_bit_cast(uint16_t, hv) | (ybits & 0x8000u);   // keep -0
      ho[i >> 1] |= hb << (16 * (i & 1));
    }
    if (active) {
      if (y) reinterpret_cast<uint4*>(y)[c] = make_uint4(yo[0], yo[1], yo[2], yo[3]);
      if (y16) reinterpret_cast<uint4*>(y16)[c] = make_uint4(ho[0], ho[1], ho[2], ho[3]);
      if (codes) reinterpret_cast<uint32_t*>(codes)[c] = packed;
      if (scales && (c & 1) == 0) scales[c / 2] = (uint8_t)scode;
    }
  }
}

static int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g > 256 * 32) g = 256 * 32;
  return g < 1 ? 1 : (int)g;
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int mxfp4_quant_1x32(const uint16_t* x, int M, int K, int64_t ldx,
                                const int32_t* row_gather, const int32_t* row_count,
                                uint8_t* codes, uint8_t* scales, void* stream) {
  FP4MOE_REQUIRE(M >= 0 && K > 0 && K % 32 == 0, "mxfp4_quant_1x32: M=%d K=%d (K %% 32 != 0)",
                 M, K);
  FP4MOE_REQUIRE(ldx >= K && ldx % 8 == 0, "mxfp4_quant_1x32: ldx=%lld", (long long)ldx);
  if (M == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(x && codes && scales, "mxfp4_quant_1x32: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)codes & 15) == 0,
                 "mxfp4_quant_1x32: x and codes must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  const int64_t blocks = (int64_t)M * (K / 32);
  hipLaunchKernelGGL(mxfp4_quant_kernel<false>, dim3(grid_for(blocks, 256)), dim3(256), 0,
                     as_stream(stream), x, M, K, ldx, row_gather, nullptr, 1, M, row_count, codes,
                     scales);
  return check_launch("mxfp4_quant_1x32");
}

extern "C" int mxfp4_quant_1x32_chunked(const uint16_t* x, int M, int K, int64_t ldx,
                                        const int32_t* row_map, int map_k, int out_rows,
                                        const int32_t* row_count, uint8_t* codes, uint8_t* scales,
                                        void* stream) {
  FP4MOE_REQUIRE(M >= 0 && K > 0 && K % 128 == 0,
                 "mxfp4_quant_1x32_chunked: M=%d K=%d (K %% 128 != 0)", M, K);
  FP4MOE_REQUIRE(ldx >= K && ldx % 8 == 0, "mxfp4_quant_1x32_chunked: ldx=%lld", (long long)ldx);
  FP4MOE_REQUIRE(row_map ? map_k >= 1 : out_rows >= M,
                 "mxfp4_quant_1x32_chunked: map_k=%d out_rows=%d M=%d", map_k, out_rows, M);
  FP4MOE_REQUIRE(out_rows >= 0, "mxfp4_quant_1x32_chunked: out_rows=%d", out_rows);
  if (M == 0 || out_rows == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(x && codes && scales, "mxfp4_quant_1x32_chunked: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)codes & 15) == 0,
                 "mxfp4_quant_1x32_chunked: x and codes must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  const int64_t blocks = (int64_t)M * (K / 32);
  hipLaunchKernelGGL(mxfp4_quant_kernel<true>, dim3(grid_for(blocks, 256)), dim3(256), 0,
                     as_stream(stream), x, M, K, ldx, nullptr, row_map, map_k, out_rows,
                     row_count, codes, scales);
  return check_launch("mxfp4_quant_1x32_chunked");
}

extern "C" int fp8_quant_per_token(const uint16_t* x, int M, int K, int64_t ldx,
                                   const int32_t* row_count, int out_rows, uint8_t* codes,
                                   float* scales, void* stream) {
  FP4MOE_REQUIRE(M >= 0 && K > 0 && K % 128 == 0 && K <= 64 * kFp8MaxSteps * 8,
                 "fp8_quant_per_token: M=%d K=%d (K a multiple of 128, at most %d)", M, K,
                 64 * kFp8MaxSteps * 8);
  FP4MOE_REQUIRE(ldx >= K && ldx % 8 == 0, "fp8_quant_per_token: ldx=%lld", (long long)ldx);
  FP4MOE_REQUIRE(out_rows >= M, "fp8_quant_per_token: out_rows=%d < M=%d", out_rows, M);
  if (M == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(x && codes && scales, "fp8_quant_per_token: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)codes & 15) == 0,
                 "fp8_quant_per_token: x and codes must be 16-byte aligned");
  FP4MOE_CHECK_DEVICE();
  const dim3 grid((unsigned)((M + 3) / 4));
  const int steps = (K / 8 + 63) / 64;
  if (steps <= 4)
    hipLaunchKernelGGL(fp8_quant_kernel<4>, grid, dim3(256), 0, as_stream(stream), x, M, K, ldx,
                       row_count, out_rows, codes, scales);
  else if (steps <= 8)
    hipLaunchKernelGGL(fp8_quant_kernel<8>, grid, dim3(256), 0, as_stream(stream), x, M, K, ldx,
                       row_count, out_rows, codes, scales);
  else
    hipLaunchKernelGGL(fp8_quant_kernel<kFp8MaxSteps>, grid, dim3(256), 0, as_stream(stream), x,
                       M, K, ldx, row_count, out_rows, codes, scales);
  return check_launch("fp8_quant_per_token");
}

extern "C" size_t nvfp4_qdq_workspace(void) { return 256; }

extern "C" int nvfp4_qdq(const uint16_t* x, int M, int K, const int32_t* row_count,
                         const float* tensor_scale_in, uint16_t* y, uint8_t* codes,
                         uint8_t* scales_e4m3, float* tensor_scale_out, uint16_t* y_f16,
                         float* y_f16_scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  FP4MOE_REQUIRE(M >= 0 && K > 0 && K % 16 == 0, "nvfp4_qdq: M=%d K=%d (K %% 16 != 0)", M, K);
  if (M == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(x && (y || y_f16), "nvfp4_qdq: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)y & 15) == 0 &&
                     ((uintptr_t)y_f16 & 15) == 0 && ((uintptr_t)codes & 3) == 0,
                 "nvfp4_qdq: x, y, y_f16 must be 16-byte and codes 4-byte aligned");
  if (!tensor_scale_in && (!workspace || workspace_bytes < nvfp4_qdq_workspace()))
    return set_error(FP4MOE_ERR_WORKSPACE, "nvfp4_qdq: dynamic scale needs %zu bytes",
                     nvfp4_qdq_workspace());
  FP4MOE_CHECK_DEVICE();
  hipStream_t s = as_stream(stream);
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  const int64_t chunks = (int64_t)M * (K / 8);
  if (!tensor_scale_in) {
    hipLaunchKernelGGL(nvfp4_zero_kernel, dim3(1), dim3(1), 0, s, ws);
    // about 16 chunks per lane, at most 1024 workgroups (atomics)
    int64_t g = (chunks + 256 * 16 - 1) / (256 * 16);
    g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)g), dim3(256), 0, s, x, M, K, row_count,
                       ws);
  }
  hipLaunchKernelGGL(nvfp4_qdq_kernel, dim3(grid_for(chunks, 256)), dim3(256), 0, s, x, M, K,
                     row_count, tensor_scale_in, ws, y, codes, scales_e4m3, tensor_scale_out,
                     y_f16, y_f16_scale);
  return check_launch("nvfp4_qdq");
}
