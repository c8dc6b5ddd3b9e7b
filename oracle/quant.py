"""Dynamic activation quantization: MXFP4 1x32 and the NVFP4 QDQ round trip.

TEST INFRASTRUCTURE ONLY (see the package docstring).

mxfp4_quant_1x32 -- [ATOM] "Stage B: Dynamic Activation Quantization" and
"From W4A8 Quark Configs to MXFP4": live bf16 activations are quantized at
run time into FP4 payloads plus one E8M0 scale per 32 values along K.  The
pages give no scale rule or rounding mode.  Reading (the OCP MX rule):
  1. amax = max |x| over the 32-block.
  2. e = floor(log2 amax) - 2   (2 = exponent of the largest E2M1 value, 6),
     clamped to [-127, 127]; the scale byte is e + 127.  amax = 0 gives e = -127.
  3. each element becomes the E2M1 code nearest to x / 2^e, ties to even,
     saturating at +-6, keeping the sign (so small negatives give code 0x8).

fp8_quant_per_token -- [GAUDI] "Exact MXFP4 to FP8 per-channel conversion":
the converted FP8 experts are served with per-channel weight scales and
dynamic per-token FP8 activations (W8A8).  The page gives no scale rule.
Reading (the plain dynamic per-row rule), in IEEE float32 like nvfp4_qdq:
  1. s_r = amax_r / 448 over the row (448 = largest OCP E4M3FN magnitude);
     s_r = 1 when the row is all zero.
  2. code = E4M3(x / s_r): one float32 division, then round to nearest even,
     saturating at +-448, sign kept.
  3. the value the GEMM sees is decode(code) * s_r (exact in float64).

nvfp4_qdq -- [NVFP4] "Weight Dequantization and Activation QDQ": activations
pass through an NVFP4 quantize-dequantize round trip before each GEMM.  The
page fixes no arithmetic.  Reading, every step an IEEE float32 operation
(round to nearest even) so that the result is reproducible bit for bit:
  1. tensor scale s_t = amax_tensor / 2688 (= 6 * 448), or the given static
     scale; s_t = 1 when the tensor is all zero.
  2. per 16-block: sb = E4M3(amax_b / f32(6 * s_t)), RNE, saturating at 448.
  3. sb == 0: all codes are zero (sign kept).  Otherwise
     code = E2M1(x / f32(sb * s_t)), RNE, saturating.
  4. y = bf16(f32(q * sb) * s_t)  where q is the E2M1 value of the code.
"""

import numpy as np

from . import formats as F

E2M1_EMAX = 2   # exponent of the largest E2M1 magnitude, 6 = 1.5 * 2^2
FP8_MAX = 448.0  # largest OCP E4M3FN magnitude


def mxfp4_quant_1x32(x_bits):
    """bf16 bit patterns [M, K] -> (codes uint8 [M, K/2], scales uint8 [M, K/32])."""
    x = F.bf16_decode(x_bits)
    M, K = x.shape
    assert K % 32 == 0
    blocks = x.reshape(M, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = F.floor_log2(amax[nz]) - E2M1_EMAX
    e = np.clip(e, -127, 127)
    q = blocks / np.ldexp(1.0, e)[..., None]   # exact: power-of-two divisor
    codes = F.e2m1_encode(q).reshape(M, K)
    return F.pack_fp4(codes), (e + 127).astype(np.uint8)


def mxfp4_qdq_values(x_bits):
    """Values the MXFP4 path feeds the GEMM: dequant(quant(x)), float64 [M, K]."""
    codes, scales = mxfp4_quant_1x32(x_bits)
    return F.mxfp4_dequant(codes, scales)


def nvfp4_qdq(x_bits, tensor_scale_in=None):
    """bf16 bits [M, K] -> dict(y bf16 bits, codes, scales (E4M3 bytes), tensor_scale)."""
    f32 = np.float32
    x = F.bf16_decode(x_bits).astype(np.float32)     # exact
    M, K = x.shape
    assert K % 16 == 0
    if tensor_scale_in is None:
        amax_t = f32(np.abs(x).max()) if x.size else f32(0)
        s_t = f32(amax_t / f32(2688.0)) if amax_t > 0 else f32(1.0)
    else:
        s_t = f32(tensor_scale_in)
    blocks = x.reshape(M, K // 16, 16)
    amax_b = np.abs(blocks).max(axis=-1).astype(np.float32)
    denom = f32(f32(6.0) * s_t)
    sb_in = (amax_b / denom).astype(np.float32)                    # f32 division
    sb = F.e4m3_round(sb_in.astype(np.float64))                     # exact E4M3 values
    sb_codes = F.e4m3_encode(sb)
    d = (sb.astype(np.float32) * s_t).astype(np.float32)            # f32 multiply
    with np.errstate(divide="ignore", invalid="ignore"):
        qin = (blocks / d[..., None]).astype(np.float32)             # f32 division
    qin = np.where((sb == 0)[..., None], np.copysign(0.0, blocks), qin)
    codes = F.e2m1_encode(qin.astype(np.float64))
    q = F.e2m1_decode(codes).astype(np.float32)
    qs = (q * sb.astype(np.float32)[..., None]).astype(np.float32)  # exact
    yv = (qs * s_t).astype(np.float32)                              # f32 multiply
    y = F.bf16_bits(yv.astype(np.float64)).reshape(M, K)
    return dict(y=y, codes=F.pack_fp4(codes.reshape(M, K)), scales=sb_codes,
                tensor_scale=float(s_t))


def fp8_quant_per_token(x_bits):
    """bf16 bit patterns [M, K] -> (E4M3 codes uint8 [M, K], scales float32 [M])."""
    f32 = np.float32
    x = F.bf16_decode(x_bits).astype(np.float32)     # exact
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = np.where(amax > 0, (amax / f32(FP8_MAX)).astype(np.float32), f32(1.0)).astype(np.float32)
    q = (x / s[:, None]).astype(np.float32)          # float32 division
    return F.e4m3_encode(q.astype(np.float64)), s


def fp8_qdq_values(x_bits):
    """Values the W8A8 path feeds the GEMM: decode(code) * s_r, float64 [M, K]."""
    codes, s = fp8_quant_per_token(x_bits)
    return F.e4m3_decode(codes) * s.astype(np.float64)[:, None]

