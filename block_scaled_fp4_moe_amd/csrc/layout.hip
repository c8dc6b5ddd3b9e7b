// fp4_weight_preshuffle: rewrite static expert weights into the fragment-major
// layout that fp4_grouped_gemm streams with 1 KiB-contiguous wave loads.
//
// [ATOM] "Stage C: MXFP4 Linear GEMM": the production FP4 GEMMs take their B
// operand pre-shuffled for the matrix instruction.  Our own layout follows the
// MFMA operand layout used by the GEMM kernels: within a 16-row group and a
// 128-wide K chunk, lane l (0..63) consumes row l % 16, 32-element block
// l / 16.  Storing those 64 lane pieces back to back makes every wave load
// one contiguous KiB (2 KiB for FP8) and every scale load one contiguous run.
//
// Layouts (G = N/16 row groups, C = K/128 chunks, f = (e*G + n/16)*C + k/128,
// h = (e*C + k/128)*G + n/16, lane = n%16 + 16*((k%128)/32)):
//   FP4 codes   byte f*1024 + lane*16 + (k%32)/2     (nibble k%2)
//   FP8 codes   byte f*2048 + ((k%32)/16)*1024 + lane*16 + k%16
//   E8M0 scale  byte h*64 + lane                      (block k/32)
//   E4M3 scale  byte h*128 + lane*2 + (k%32)/16       (block k/16)
// Codes are group-major (a group's chunks follow each other); scales are
// chunk-major, so one chunk's scales of consecutive row groups are one run.
// FP8 channel scales keep their [E, N] layout.
#include "common.h"

namespace fp4moe {

// One thread per output 16-byte piece (FP4/FP8 codes) or per scale byte.
__global__ __launch_bounds__(256) void shuffle_codes_kernel(const uint8_t* __restrict__ in,
                                                            uint8_t* __restrict__ out, int64_t E,
                                                            int N, int K, int bytes_per_block) {
  // bytes_per_block: 16 (FP4: 32 elements) or 32 (FP8)
  const int C = K / 128, G = N / 16;
  const int64_t pieces_per_frag = 64 * (bytes_per_block / 16);
  const int64_t total = E * G * C * pieces_per_frag;
  const int64_t row_bytes = (int64_t)(K / 32) * bytes_per_block;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = i / pieces_per_frag;
    const int piece = (int)(i - f * pieces_per_frag);
    const int half = piece / 64, lane = piece % 64;
    const int c = (int)(f % C);
    const int64_t eg = f / C;
    const int grp = (int)(eg % G);
    const int64_t e = eg / G;
    const int n = grp * 16 + (lane & 15);
    const int blk = c * 4 + (lane >> 4);
    const int64_t src = (e * N + n) * row_bytes + (int64_t)blk * bytes_per_block + half * 16;
    reinterpret_cast<uint4*>(out)[i] = *reinterpret_cast<const uint4*>(in + src);
  }
}

__global__ __launch_bounds__(256) void shuffle_scales_kernel(const uint8_t* __restrict__ in,
                                                             uint8_t* __restrict__ out, int64_t E,
                                                             int N, int K, int per_block) {
  // per_block: 1 (E8M0 per 32) or 2 (E4M3 per 16) scale bytes per 32-element block
  const int C = K / 128, G = N / 16;
  const int64_t per_frag = 64 * per_block;
  const int64_t total = E * G * C * per_frag;
  const int64_t row_bytes = (int64_t)(K / 32) * per_block;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = i / per_frag;                 // (e*C + c)*G + grp
    const int j = (int)(i - h * per_frag);
    const int lane = j / per_block, sub = j % per_block;
    const int grp = (int)(h % G);
    const int64_t ec = h / G;
    const int c = (int)(ec % C);
    const int64_t e = ec / C;
    const int n = grp * 16 + (lane & 15);
    const int blk = c * 4 + (lane >> 4);
    out[i] = in[(e * N + n) * row_bytes + (int64_t)blk * per_block + sub];
  }
}

static unsigned shuffle_grid(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 256 * 64) g = 256 * 64;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace fp4moe

using namespace fp4moe;

extern "C" int fp4_weight_preshuffle(int wfmt, int E, int N, int K, const uint8_t* codes,
                                     const uint8_t* scales, uint8_t* codes_out,
                                     uint8_t* scales_out, void* stream) {
  FP4MOE_REQUIRE(wfmt == FP4MOE_W_MXFP4 || wfmt == FP4MOE_W_NVFP4 || wfmt == FP4MOE_W_FP8,
                 "fp4_weight_preshuffle: wfmt=%d", wfmt);
  FP4MOE_REQUIRE(E >= 0 && N > 0 && N % 16 == 0 && K > 0 && K % 128 == 0,
                 "fp4_weight_preshuffle: E=%d N=%d K=%d (N %% 16, K %% 128)", E, N, K);
  if (E == 0) return FP4MOE_OK;
  FP4MOE_REQUIRE(codes && codes_out && codes != codes_out,
                 "fp4_weight_preshuffle: codes must be distinct non-null buffers");
  FP4MOE_REQUIRE(((uintptr_t)codes & 15) == 0 && ((uintptr_t)codes_out & 15) == 0,
                 "fp4_weight_preshuffle: code buffers must be 16-byte aligned");
  FP4MOE_REQUIRE(wfmt == FP4MOE_W_FP8 || (scales && scales_out && scales != scales_out),
                 "fp4_weight_preshuffle: scales must be distinct non-null buffers");
  FP4MOE_CHECK_DEVICE();
  hipStream_t s = as_stream(stream);
  const int bpb = (wfmt == FP4MOE_W_FP8) ? 32 : 16;
  const int64_t pieces = (int64_t)E * (N / 16) * (K / 128) * 64 * (bpb / 16);
  hipLaunchKernelGGL(shuffle_codes_kernel, dim3(shuffle_grid(pieces)), dim3(256), 0, s, codes,
                     codes_out, (int64_t)E, N, K, bpb);
  if (wfmt != FP4MOE_W_FP8) {
    const int per = (wfmt == FP4MOE_W_MXFP4) ? 1 : 2;
    const int64_t n_sc = (int64_t)E * N * (K / 32) * per;
    hipLaunchKernelGGL(shuffle_scales_kernel, dim3(shuffle_grid(n_sc)), dim3(256), 0, s, scales,
                       scales_out, (int64_t)E, N, K, per);
  }
  return check_launch("fp4_weight_preshuffle");
}
