"""CPU oracle for the block-scaled FP4 routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition of every step of the layer, written in NumPy with float64
arithmetic (or IEEE float32 where the method fixes that precision).  It exists
so that the HIP library can be checked against it.  Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the HIP library and its Python binding) never does, and shares no code,
table or helper with it.

Sources (web pages, cited by title and section):
  [ATOM]   "Serve Kimi-K2.5-MXFP4 on MI355X with ATOM" (ROCm blog)
  [NVFP4]  "Serving NVFP4 models on AMD Instinct MI355 accelerators"
  [GAUDI]  "Kimi-K2.7-Code on Gaudi 2" (gaudi-cookbook port notes)
  [K3]     "Kimi K3 on MI355X" (vLLM blog mirror)

Modules
  formats   E2M1 / E8M0 / E4M3 / bf16 encodings and round-to-nearest-even
  route     grouped sigmoid top-k routing with a correction bias
  permute   stable sort of (token, slot) pairs by expert, tile list
  quant     dynamic 1x32 MXFP4 activation quantization, NVFP4 QDQ
  gemm      grouped expert GEMMs (gate/up + SiLU*up, down) and the combine
  convert   exact MXFP4 -> FP8 E4M3 per-channel conversion
  layer     the whole layer chained from the steps above

Parity pins for every function live in tests/test_oracle_*.py (CPU only).
"""

from . import formats, route, permute, quant, gemm, convert, layer  # noqa: F401
