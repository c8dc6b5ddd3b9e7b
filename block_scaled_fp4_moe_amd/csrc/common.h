// Internal helpers shared by the fp4moe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4moe.h"

namespace fp4moe {

// ---- host-side status handling -------------------------------------------

int set_error(int status, const char* fmt, ...);   // records a thread-local message
int check_device();                                 // FP4MOE_OK on gfx950
int check_launch(const char* what);                 // maps hipGetLastError to a status

#define FP4MOE_REQUIRE(cond, ...)                                          \
  do {                                                                     \
    if (!(cond)) return ::fp4moe::set_error(FP4MOE_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

#define FP4MOE_CHECK_DEVICE()                 \
  do {                                        \
    int _st = ::fp4moe::check_device();       \
    if (_st != FP4MOE_OK) return _st;         \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---- device helpers ------------------------------------------------------

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bit pattern, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// E2M1 code magnitude (0..7) of |q| by round-to-nearest-even on the grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6: ties 0.25, 1.25, 2.5, 5 go
// down and 0.75, 1.75, 3.5 go up, always to the even code.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// E2M1 codes of eight bf16 values (four words, element 2i in the low half)
// times the power of two inv, packed element i at nibble i.  The gfx950
// float -> E2M1 conversion rounds exactly as e2m1_mag_code (nearest, ties to
// even, saturating at 6, sign kept; checked on the device for every finite
// bf16 pattern at several scalings, denormals included), so it does the work
// when no value is NaN; NaN values take the compare path (code 0, sign kept).
__device__ __forceinline__ uint32_t e2m1_pack8(const uint32_t w[4], float inv, bool has_nan) {
  if (!has_nan) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(w[0] << 16) * inv,
                                                 __uint_as_float(w[0] & 0xffff0000u) * inv, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(w[1] << 16) * inv,
                                                 __uint_as_float(w[1] & 0xffff0000u) * inv, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(w[2] << 16) * inv,
                                                 __uint_as_float(w[2] & 0xffff0000u) * inv, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(w[3] << 16) * inv,
                                                 __uint_as_float(w[3] & 0xffff0000u) * inv, 1.0f, 3);
    return r;
  }
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
    packed |= (e2m1_mag_code(bf16_to_f32(h & 0x7fffu) * inv) | ((h >> 12) & 8u)) << (4 * i);
  }
  return packed;
}

// 2^e as a float for e in [-126, 127] (normal range).
__device__ __forceinline__ float exp2i(int e) {
  return __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
}

// E8M0 byte -> float scale 2^(c-127) (c = 0 gives the subnormal 2^-127; 255 -> NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  if (c == 0) return __uint_as_float(0x00400000u);
  if (c == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(c << 23);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace fp4moe
