// mxfp4_to_fp8_channel: exact MXFP4 -> FP8 E4M3 per-channel conversion.
//
// [GAUDI] "Exact MXFP4 to FP8 per-channel conversion".  For a row x of
// decoded MXFP4 values:  e_max = floor(log2 max_i |x_i|),  k = e_max - 7,
// channel scale = 2^k,  code_i = E4M3(x_i * 2^-k).  If the row's E8M0 codes
// lie within 9 consecutive binades, every x_i * 2^-k is 0 or a normal E4M3
// value with exponent in [-5, 7] (magnitude <= 1.5 * 2^7), so
// decode(code_i) * 2^k == x_i for every element.
//
// The kernel is integer-only.  One wavefront converts one row in two passes
// over its blocks (all of the row's codes held in registers):
//   pass 1: the largest element exponent of a block is its E8M0 exponent plus
//           the exponent class of its largest E2M1 magnitude, found with a few
//           bit tests on the packed nibbles; a wavefront max gives e_max.
//   pass 2: within a block every element with magnitude code c maps to the
//           same FP8 byte (sign aside), so the block's 8-entry byte table is
//           built once and applied to 4 nibbles per v_perm_b32.
#include "common.h"

namespace fp4moe {

constexpr int kNoElement = -100000;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Exponent class of the largest magnitude among the 8 nibbles of each word:
// codes 6,7 -> 2; 4,5 -> 1; 2,3 -> 0; 1 -> -1; none -> kNoElement.
__device__ __forceinline__ int block_max_class(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t m0 = w0 & 0x77777777u, m1 = w1 & 0x77777777u, m2 = w2 & 0x77777777u,
                 m3 = w3 & 0x77777777u;
  const uint32_t any = m0 | m1 | m2 | m3;
  const uint32_t six = ((m0 & (m0 << 1)) | (m1 & (m1 << 1)) | (m2 & (m2 << 1)) |
                        (m3 & (m3 << 1))) & 0x44444444u;
  if (six) return 2;
  if (any & 0x44444444u) return 1;
  if (any & 0x22222222u) return 0;
  if (any & 0x11111111u) return -1;
  return kNoElement;
}

// The same for half a block (16 nibbles in two words).
__device__ __forceinline__ int half_max_class(uint32_t w0, uint32_t w1) {
  return block_max_class(w0, w1, 0u, 0u);
}

// FP8 byte of the E2M1 magnitude code c (1..7) scaled by 2^d, with flags.
// value = sig * 2^(cls + d), sig in {1, 1.5}.
__device__ __forceinline__ uint32_t fp8_of_mag(int c, int d, bool* inexact, bool* below) {
  const int cls = (c >> 1) - 1;           // 1 -> -1, 2,3 -> 0, 4,5 -> 1, 6,7 -> 2
  const bool half = (c == 3) || (c == 5) || (c == 7);
  const int E = cls + d;
  *below = E < -5;
  *inexact = false;
  if (E >= -6) return ((uint32_t)(E + 7) << 3) | (half ? 4u : 0u);
  // E4M3 subnormal: value in units of 2^-9, round half to even.
  const int sh = E + 9;                   // units = sig * 2^sh, sh <= 2
  if (sh <= -2) {                         // below a quarter unit: rounds to zero
    *inexact = true;
    return 0u;
  }
  float units = (half ? 1.5f : 1.0f) * ldexpf(1.0f, sh);
  const float r = rintf(units);
  *inexact = (r != units);
  return (uint32_t)r;
}

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

// Encode 16 values of a block (codes w0, w1; E8M0 byte s, d = s - 127 - k)
// into 16 FP8 bytes; sets the below / inexact flags for elements that need
// them.  Every value with magnitude code c maps to the same byte (sign
// aside), so an 8-entry byte table is built once and applied to 4 nibbles
// per v_perm_b32.
__device__ __forceinline__ uint4 encode_half(uint32_t w0, uint32_t w1, int s, int k,
                                             bool* any_below, bool* any_inexact) {
  const int d = s - 127 - k;
  uint32_t lut_lo = 0, lut_hi = 0;
  uint32_t below_mask = 0, inexact_mask = 0;
  if (d >= -4) {
    // fast path: every class lands on a normal with exponent >= -5, exact
#pragma unroll
    for (int c = 1; c < 8; ++c) {
      const int cls = (c >> 1) - 1;
      const uint32_t byte = ((uint32_t)(cls + d + 7) << 3) | ((c & 1) && c > 1 ? 4u : 0u);
      if (c < 4) lut_lo |= byte << (8 * c);
      else lut_hi |= byte << (8 * (c - 4));
    }
  } else {
#pragma unroll
    for (int c = 1; c < 8; ++c) {
      bool inex, below;
      const uint32_t byte = fp8_of_mag(c, d, &inex, &below);
      if (c < 4) lut_lo |= byte << (8 * c);
      else lut_hi |= byte << (8 * (c - 4));
      below_mask |= (below ? 1u : 0u) << c;
      inexact_mask |= (inex ? 1u : 0u) << c;
    }
  }
  const uint32_t win[2] = {w0, w1};
  uint32_t out[4];
  uint32_t present = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // bytes [b0,b0,b1,b1] and [b2,b2,b3,b3], then keep lo/hi nibble alternately
    const uint32_t t0 = __builtin_amdgcn_perm(win[i], win[i], 0x01010000u);
    const uint32_t t1 = __builtin_amdgcn_perm(win[i], win[i], 0x03030202u);
    const uint32_t x0 = (t0 & 0x000f000fu) | ((t0 >> 4) & 0x0f000f00u);
    const uint32_t x1 = (t1 & 0x000f000fu) | ((t1 >> 4) & 0x0f000f00u);
    out[2 * i] = __builtin_amdgcn_perm(lut_hi, lut_lo, x0 & 0x07070707u) |
                 ((x0 & 0x08080808u) << 4);
    out[2 * i + 1] = __builtin_amdgcn_perm(lut_hi, lut_lo, x1 & 0x07070707u) |
                     ((x1 & 0x08080808u) << 4);
    if (below_mask | inexact_mask) {
#pragma unroll
      for (int n = 0; n < 8; ++n) present |= 1u << ((win[i] >> (4 * n)) & 7u);
    }
  }
  *any_below |= (present & below_mask) != 0;
  *any_inexact |= (present & inexact_mask) != 0;
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// One wavefront per row, each lane owning half blocks (16 values: 8 code
// bytes in, 16 FP8 bytes out), so that every load and store instruction of
// the wavefront covers one contiguous run.  The row's codes and scales stay
// in registers between the two passes (NH half blocks per lane,
// K <= 1024 * NH), and the FP8 bytes are written with streaming stores.
template <int NH>
__global__ __launch_bounds__(256) void mx_to_fp8_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        int64_t rows, int K,
                                                        uint8_t* __restrict__ fp8,
                                                        float* __restrict__ channel_scale,
                                                        uint8_t* __restrict__ row_status,
                                                        uint32_t* __restrict__ n_inexact) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nhalf = K / 16;
  const uint8_t* crow = codes + row * (K / 2);
  const uint8_t* srow = scales + row * (K / 32);
  uint8_t* orow = fp8 + row * K;

  uint2 w[NH];
  int sc[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int hb = lane + 64 * j;
    sc[j] = 255;
    w[j] = make_uint2(0, 0);
    if (hb < nhalf) {
      sc[j] = srow[hb >> 1];
      w[j] = *reinterpret_cast<const uint2*>(crow + hb * 8);
    }
  }
  // pass 1: e_max over finite blocks
  int emax = kNoElement;
  bool has_nan = false;
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    if (lane + 64 * j >= nhalf) continue;
    if (sc[j] == 255) {
      has_nan = true;
      continue;
    }
    const int cls = half_max_class(w[j].x, w[j].y);
    if (cls != kNoElement) emax = max(emax, sc[j] - 127 + cls);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) emax = max(emax, __shfl_xor(emax, off, 64));
  const bool zero_row = (emax == kNoElement);
  const int k = zero_row ? 0 : emax - 7;

  // pass 2: encode
  bool any_below = false, any_inexact = false;
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int hb = lane + 64 * j;
    if (hb >= nhalf) continue;
    uint4 o;
    if (sc[j] == 255) {
      o = make_uint4(0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu);
    } else {
      o = encode_half(w[j].x, w[j].y, sc[j], k, &any_below, &any_inexact);
    }
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4*>(orow + hb * 16));
  }
  has_nan = __ballot(has_nan) != 0;
  any_below = __ballot(any_below) != 0;
  any_inexact = __ballot(any_inexact) != 0;
  if (lane == 0) {
    channel_scale[row] = ldexpf(1.0f, k);
    if (row_status) {
      row_status[row] = has_nan ? 2 : (zero_row ? 3 : (any_below ? 1 : 0));
    }
    if (any_inexact) atomicAdd(n_inexact, 1u);
  }
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int mxfp4_to_fp8_channel(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                    int K, uint8_t* fp8, float* channel_scale,
                                    uint8_t* row_status, uint32_t* n_inexact_rows, void* stream) {
  FP4MOE_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0,
                 "mxfp4_to_fp8_channel: rows=%lld K=%d (K %% 32 != 0)", (long long)rows, K);
  FP4MOE_REQUIRE(n_inexact_rows, "mxfp4_to_fp8_channel: n_inexact_rows is required");
  FP4MOE_REQUIRE(rows == 0 || (codes && scales && fp8 && channel_scale),
                 "mxfp4_to_fp8_channel: null pointer");
  FP4MOE_REQUIRE(((uintptr_t)codes & 15) == 0 && ((uintptr_t)fp8 & 15) == 0,
                 "mxfp4_to_fp8_channel: codes and fp8 must be 16-byte aligned");
  FP4MOE_REQUIRE((rows + 3) / 4 < (1ll << 31), "mxfp4_to_fp8_channel: too many rows");
  FP4MOE_REQUIRE(K <= 2048 * 16, "mxfp4_to_fp8_channel: K=%d above 32768", K);
  FP4MOE_CHECK_DEVICE();
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, n_inexact_rows);
  if (rows > 0) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const int nh = (K / 16 + 63) / 64;     // half blocks per lane
#define FP4MOE_CONVERT(NH)                                                                       \
  hipLaunchKernelGGL(mx_to_fp8_kernel<NH>, grid, block, 0, s, codes, scales, rows, K, fp8,       \
                     channel_scale, row_status, n_inexact_rows)
    if (nh <= 1) FP4MOE_CONVERT(1);
    else if (nh <= 2) FP4MOE_CONVERT(2);
    else if (nh <= 4) FP4MOE_CONVERT(4);
    else if (nh <= 8) FP4MOE_CONVERT(8);
    else if (nh <= 16) FP4MOE_CONVERT(16);
    else FP4MOE_CONVERT(32);
#undef FP4MOE_CONVERT
  }
  return check_launch("mxfp4_to_fp8_channel");
}
