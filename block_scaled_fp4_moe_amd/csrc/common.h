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
