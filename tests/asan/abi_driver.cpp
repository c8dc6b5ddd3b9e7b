// Host-side argument validation of every C-ABI entry point, run under
// AddressSanitizer (host code instrumented; no GPU is needed or touched).
//
// Every "device" pointer handed to the library is the address of a freed
// heap block: the validation may look at the address (null, alignment) but
// must never read through it, and AddressSanitizer reports any read as a
// use-after-free.  Each call is checked for its status, and the message of
// fp4moe_last_error() is read in full after it.  Calls whose arguments are
// valid stop at the device check (no gfx950 device here) and must not return
// FP4MOE_ERR_INVALID_ARG.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fp4moe.h"

static int g_fail = 0;
static int g_calls = 0;

enum Want { BAD = 0, OK = 1, VALID = 2 };   // invalid argument / OK / anything but invalid

static void check(int line, const char* what, int st, Want want) {
  ++g_calls;
  const char* msg = fp4moe_last_error();
  const size_t n = strlen(msg);   // the whole message is read (ASan checks the buffer)
  bool good = want == BAD ? st == FP4MOE_ERR_INVALID_ARG
            : want == OK  ? st == FP4MOE_OK
                          : st != FP4MOE_ERR_INVALID_ARG;
  if (want == BAD && n == 0) good = false;   // an error always says why
  if (!good) {
    fprintf(stderr, "line %d: %s -> %d (%s)\n", line, what, st, msg);
    ++g_fail;
  }
}
#define EXPECT(call, want) check(__LINE__, #call, (call), (want))

int main() {
  // a freed 4 KiB block, 256-byte aligned: the stand-in for device memory
  void* block = nullptr;
  if (posix_memalign(&block, 256, 4096) != 0) return 2;
  free(block);
  char* D = static_cast<char*>(block);
  auto F = reinterpret_cast<float*>(D);
  auto I32 = reinterpret_cast<int32_t*>(D);
  auto U16 = reinterpret_cast<uint16_t*>(D);
  auto U8 = reinterpret_cast<uint8_t*>(D);
  auto U32 = reinterpret_cast<uint32_t*>(D);

  EXPECT(fp4moe_init(), VALID);

  // routing
  EXPECT(moe_route(F, F, 8, 384, 8, 4, 8, 1, 1.f, I32, F, nullptr), VALID);
  EXPECT(moe_route(F, F, -1, 384, 8, 4, 8, 1, 1.f, I32, F, nullptr), BAD);
  EXPECT(moe_route(F, F, 8, 2000, 8, 4, 8, 1, 1.f, I32, F, nullptr), BAD);
  EXPECT(moe_route(F, F, 8, 384, 7, 4, 8, 1, 1.f, I32, F, nullptr), BAD);
  EXPECT(moe_route(F, F, 8, 384, 8, 9, 8, 1, 1.f, I32, F, nullptr), BAD);
  EXPECT(moe_route(F, F, 8, 384, 8, 4, 33, 1, 1.f, I32, F, nullptr), BAD);
  EXPECT(moe_route(nullptr, F, 8, 384, 8, 4, 8, 1, 1.f, I32, F, nullptr), BAD);

  // permutation
  EXPECT(moe_permute_max_tiles(8, 8, 384, 1, 16) > 0 ? FP4MOE_OK : -1, OK);
  const size_t ws = moe_permute_workspace(4096, 8, 384, 1, 16);
  EXPECT(moe_permute(I32, 8, 8, 384, 1, 16, nullptr, 0, I32, I32, I32, I32, I32, I32, nullptr),
         VALID);
  EXPECT(moe_permute(I32, 4096, 8, 384, 1, 16, D, ws, I32, I32, I32, I32, I32, I32, nullptr),
         VALID);
  EXPECT(moe_permute(I32, 4096, 8, 384, 1, 16, D, ws - 4, I32, I32, I32, I32, I32, I32, nullptr) ==
                 FP4MOE_ERR_WORKSPACE ? FP4MOE_OK : -1, OK);
  EXPECT(moe_permute(I32, 8, 0, 384, 1, 16, nullptr, 0, I32, I32, I32, I32, I32, I32, nullptr), BAD);
  EXPECT(moe_permute(I32, 8, 8, 384, 9, 16, nullptr, 0, I32, I32, I32, I32, I32, I32, nullptr), BAD);
  EXPECT(moe_permute(I32, 8, 8, 384, 1, 2048, nullptr, 0, I32, I32, I32, I32, I32, I32, nullptr),
         BAD);
  EXPECT(moe_permute(I32, 8, 8, 384, 1, 16, nullptr, 0, nullptr, I32, I32, I32, I32, I32, nullptr),
         BAD);
  EXPECT(moe_permute_noalloc_max_workspace() > 0 ? FP4MOE_OK : -1, OK);
  EXPECT(moe_permute_noalloc(I32, 64, 8, 384, 1, 16, I32, I32, I32, I32, I32, I32, nullptr), VALID);
  EXPECT(moe_permute_noalloc(I32, 3000000, 8, 384, 1, 16, I32, I32, I32, I32, I32, I32, nullptr) ==
                 FP4MOE_ERR_WORKSPACE ? FP4MOE_OK : -1, OK);
  EXPECT(moe_route_permute(F, F, 8, 384, 8, 4, 8, 1, 1.f, 1, 16, I32, F, I32, I32, I32, I32, I32,
                           I32, nullptr), VALID);
  EXPECT(moe_route_permute(F, F, 200, 384, 8, 4, 8, 1, 1.f, 1, 16, I32, F, I32, I32, I32, I32,
                           I32, I32, nullptr), BAD);   // more than 1024 pairs

  // quantization
  EXPECT(mxfp4_quant_1x32(U16, 8, 7168, 7168, nullptr, nullptr, U8, U8, nullptr), VALID);
  EXPECT(mxfp4_quant_1x32(U16, 8, 7000, 7168, nullptr, nullptr, U8, U8, nullptr), BAD);
  EXPECT(mxfp4_quant_1x32(U16, 8, 7168, 7000, nullptr, nullptr, U8, U8, nullptr), BAD);
  EXPECT(mxfp4_quant_1x32_chunked(U16, 8, 7168, 7168, I32, 9, 72, nullptr, U8, U8, nullptr), VALID);
  EXPECT(mxfp4_quant_1x32_chunked(U16, 8, 7100, 7168, I32, 9, 72, nullptr, U8, U8, nullptr), BAD);
  EXPECT(fp8_quant_per_token(U16, 8, 7168, 7168, nullptr, 8, U8, F, nullptr), VALID);
  EXPECT(fp8_quant_per_token(U16, 8, 7168, 7168, nullptr, 4, U8, F, nullptr), BAD);
  EXPECT(fp8_quant_per_token(U16, 8, 100, 7168, nullptr, 8, U8, F, nullptr), BAD);
  EXPECT(nvfp4_qdq(U16, 8, 7168, nullptr, nullptr, U16, nullptr, nullptr, nullptr, nullptr,
                   nullptr, D, nvfp4_qdq_workspace(), nullptr), VALID);
  EXPECT(nvfp4_qdq(U16, 8, 7160, nullptr, nullptr, U16, nullptr, nullptr, nullptr, nullptr,
                   nullptr, D, nvfp4_qdq_workspace(), nullptr), BAD);
  EXPECT(nvfp4_qdq(U16, 8, 7168, nullptr, nullptr, U16, nullptr, nullptr, nullptr, nullptr,
                   nullptr, nullptr, 0, nullptr) == FP4MOE_ERR_WORKSPACE ? FP4MOE_OK : -1, OK);

  // grouped GEMM
  fp4moe_gemm_args g;
  memset(&g, 0, sizeof(g));
  g.stage = 1; g.wfmt = FP4MOE_W_MXFP4; g.afmt = FP4MOE_A_BF16; g.n_experts = 385;
  g.N = 4096; g.K = 7168; g.max_rows = 72; g.max_tiles = 72; g.block_m = 16; g.gather_div = 9;
  g.w = U8; g.w_scale = U8; g.a = D; g.lda = 7168; g.a_row_gather = I32;
  g.expert_offsets = I32; g.tiles = I32; g.n_tiles = I32; g.out = U16; g.ldo = 2048;
  g.w_layout = FP4MOE_LAYOUT_FRAGMENT;
  EXPECT(fp4_grouped_gemm(&g, nullptr), VALID);
  EXPECT(fp4_grouped_gemm(nullptr, nullptr), BAD);
  { fp4moe_gemm_args b = g; b.stage = 3; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.K = 100; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.block_m = 48; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.ldo = 100; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.w = U8 + 4; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.afmt = FP4MOE_A_F16; b.wfmt = FP4MOE_W_NVFP4; b.block_m = 128;
    b.K = 7168; b.w_tensor_scale = F; b.a_f16_scale = F; b.work_queue = I32;
    EXPECT(fp4_grouped_gemm(&b, nullptr), VALID);
    b.work_queue = reinterpret_cast<int32_t*>(D + 2); EXPECT(fp4_grouped_gemm(&b, nullptr), BAD);
    b.work_queue = I32; b.K = 7040; b.lda = 7040; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  { fp4moe_gemm_args b = g; b.afmt = FP4MOE_A_MXFP4; b.block_m = 192; b.N = 4096; b.ldo = 2048;
    b.a_scale = U8; b.a_layout = FP4MOE_A_LAYOUT_CHUNKED; b.a_rows = 72; b.a_row_gather = nullptr;
    EXPECT(fp4_grouped_gemm(&b, nullptr), VALID);
    b.out_q = U8; EXPECT(fp4_grouped_gemm(&b, nullptr), BAD); }
  EXPECT(mxfp4_linear(U8, U8, 16384, 7168, 1, 16384, U8, U8, 7168, U16, 7168, nullptr, nullptr),
         VALID);
  EXPECT(mxfp4_linear(U8, U8, 16384, 7100, 1, 16384, U8, U8, 7168, U16, 7168, nullptr, nullptr),
         BAD);
  EXPECT(fp4_weight_preshuffle(FP4MOE_W_MXFP4, 2, 4096, 7168, U8, U8, U8 + 2048, U8 + 3072,
                               nullptr), VALID);
  EXPECT(fp4_weight_preshuffle(FP4MOE_W_MXFP4, 2, 24, 256, U8, U8, U8, U8, nullptr), BAD);

  // combine, fused decode, conversion
  EXPECT(moe_combine(U16, I32, F, 8, 8, 1, 7168, U16, nullptr, nullptr), VALID);
  EXPECT(moe_combine(U16, I32, F, 8, 8, 1, 7164, U16, nullptr, nullptr), BAD);
  EXPECT(moe_combine(U16 + 1, I32, F, 8, 8, 1, 7168, U16, nullptr, nullptr), BAD);
  fp4moe_decode_args d;
  memset(&d, 0, sizeof(d));
  d.T = 8; d.H = 7168; d.I = 2048; d.E = 384; d.n_shared = 1; d.n_group = 8; d.topk_group = 4;
  d.topk = 8; d.renormalize = 1; d.max_tiles = 72; d.routed_scale = 1.f;
  d.x = U16; d.logits = F; d.w13 = U8; d.w13_scale = U8; d.w2 = U8; d.w2_scale = U8;
  d.topk_ids = I32; d.topk_w = F; d.expert_offsets = I32; d.sorted_pairs = I32; d.pair_pos = I32;
  d.tiles = I32; d.n_tiles = I32; d.n_dropped = I32; d.h = U16; d.y = U16; d.out = U16;
  d.workspace = D; d.workspace_bytes = moe_decode_fused_workspace(7168);
  EXPECT(moe_decode_fused(&d, nullptr), VALID);
  { fp4moe_decode_args b = d; b.T = 17; EXPECT(moe_decode_fused(&b, nullptr), BAD); }
  { fp4moe_decode_args b = d; b.workspace_bytes = 4;
    EXPECT(moe_decode_fused(&b, nullptr) == FP4MOE_ERR_WORKSPACE ? FP4MOE_OK : -1, OK); }
  EXPECT(mxfp4_to_fp8_channel(U8, U8, 4096, 7168, U8, F, U8, U32, nullptr), VALID);
  EXPECT(mxfp4_to_fp8_channel(U8, U8, 4096, 7100, U8, F, U8, U32, nullptr), BAD);
  EXPECT(mxfp4_to_fp8_channel(U8, U8, -1, 7168, U8, F, U8, U32, nullptr), BAD);

  EXPECT(moe_route(F, F, 8, 384, 8, 4, 8, 1, 1.f, nullptr, F, nullptr), BAD);

  printf("%d calls, %d failures\n", g_calls, g_fail);
  return g_fail == 0 ? 0 : 1;
}
