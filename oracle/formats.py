"""Number formats used by the layer, decoded and encoded in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[ATOM] "MXFP4 Tensor Anatomy": an MXFP4 tensor is a payload of FP4 E2M1
values packed two per uint8 byte plus one E8M0 scale byte per 32 values along
K; 16 + 1 bytes per 32 values.  [ATOM] "The Kimi-K2.5-MXFP4 Model on gfx950":
the E8M0 scale is a shared power-of-two exponent for the block.

The pages do not print the E2M1 value table, the nibble order or the E8M0
bias.  Readings (each pinned by tests/test_oracle_formats.py):
  * E2M1 code bits are s e1 e0 m; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
    [GAUDI] "Exact MXFP4 to FP8 per-channel conversion" fixes the largest
    significand at 1.5 (an element with k = e_max - 7 never exceeds 192 =
    1.5 * 2^7), consistent with this table.
  * Element 2i sits in the low nibble of byte i, element 2i+1 in the high one.
  * E8M0 code c means 2^(c - 127); code 255 is NaN.
  * E4M3 is the OCP E4M3FN encoding: bias 7, no infinities, 0x7F/0xFF NaN,
    largest finite 448.  For exponents -6..7 its bit patterns coincide with
    the IEEE-style E4M3 of [GAUDI] (largest finite 240).
"""

import numpy as np

# Magnitudes of the eight non-negative E2M1 codes, indexed by (code & 7).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
BF16_MAX = float(np.ldexp(255.0, 120))  # (2 - 2^-7) * 2^127


# --------------------------------------------------------------------------
# Packing
# --------------------------------------------------------------------------

def unpack_fp4(packed):
    """uint8 [..., K/2] -> 4-bit codes uint8 [..., K]; low nibble first."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_fp4(codes):
    """4-bit codes uint8 [..., K] -> uint8 [..., K/2]; element 2i in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 0x0F) | ((codes[..., 1::2] & 0x0F) << 4)


# --------------------------------------------------------------------------
# Decoding by table lookup
# --------------------------------------------------------------------------

def e2m1_decode(codes):
    """4-bit E2M1 codes -> float64 (sign bit 3; code 0x8 is -0.0)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


def e8m0_decode(scales):
    """E8M0 bytes -> float64 2^(c-127); 255 -> NaN."""
    s = np.asarray(scales, dtype=np.int64)
    val = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, val)


def e4m3_decode(codes):
    """OCP E4M3FN bytes -> float64.  0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    normal = np.ldexp(1.0 + mf / 8.0, ef - 7)
    sub = np.ldexp(mf / 8.0, -6)
    mag = np.where(ef == 0, sub, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def bf16_decode(bits):
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def mxfp4_dequant(packed, scales):
    """MXFP4 [..., K/2] codes + [..., K/32] E8M0 scales -> float64 [..., K]."""
    v = e2m1_decode(unpack_fp4(packed))
    K = v.shape[-1]
    s = e8m0_decode(scales)
    assert s.shape[-1] * 32 == K
    return v * np.repeat(s, 32, axis=-1)


def nvfp4_dequant(packed, scales_e4m3, tensor_scale):
    """NVFP4 [..., K/2] codes, [..., K/16] E4M3 scales, float tensor scale -> float64."""
    v = e2m1_decode(unpack_fp4(packed))
    s = e4m3_decode(scales_e4m3)
    assert s.shape[-1] * 16 == v.shape[-1]
    return v * np.repeat(s, 16, axis=-1) * float(tensor_scale)


# --------------------------------------------------------------------------
# Round to nearest, ties to even, onto a binary floating-point grid
# --------------------------------------------------------------------------

def round_to_grid(x, mbits, emin, maxval, saturate):
    """Round float64 x to the nearest value of a binary float format.

    The format has `mbits` explicit significand bits, smallest normal exponent
    `emin` (subnormals continue with the emin quantum) and largest finite
    magnitude `maxval`.  Ties go to the even significand.  Magnitudes beyond
    maxval become maxval if `saturate`, else infinity.  The sign of the input
    is kept, also when the result is zero.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)            # a = m * 2^ex with m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, emin)   # floor(log2 a), clamped
    quantum = np.ldexp(1.0, e - mbits)
    r = np.rint(a / quantum) * quantum  # np.rint rounds half to even
    r = np.where(a == 0, 0.0, r)
    if saturate:
        r = np.where(r > maxval, maxval, r)
    else:
        r = np.where(r > maxval, np.inf, r)
    return np.copysign(r, x)


def e2m1_encode(x):
    """float64 -> 4-bit E2M1 codes, RNE, saturating at +-6, sign kept."""
    r = round_to_grid(x, mbits=1, emin=0, maxval=E2M1_MAX, saturate=True)
    mag = np.abs(r)
    idx = np.searchsorted(E2M1_MAGNITUDES, mag)
    assert np.all(E2M1_MAGNITUDES[np.clip(idx, 0, 7)] == mag)
    return (idx.astype(np.uint8) | np.where(np.signbit(r), 8, 0).astype(np.uint8)).astype(np.uint8)


def e4m3_encode(x):
    """float64 -> OCP E4M3FN bytes, RNE, saturating at +-448, sign kept."""
    r = round_to_grid(x, mbits=3, emin=-6, maxval=E4M3_MAX, saturate=True)
    a = np.abs(r)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1
    normal = a >= 2.0 ** -6
    ef = np.where(normal, e + 7, 0)
    mf_norm = np.where(normal, np.ldexp(a, -np.where(normal, e, 0)) * 8 - 8, 0)
    mf_sub = a / 2.0 ** -9
    mf = np.where(normal, mf_norm, mf_sub)
    code = (ef.astype(np.int64) << 3) | mf.astype(np.int64)
    code = np.where(a == 0, 0, code)
    code = code | np.where(np.signbit(r), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_round(x):
    """float64 -> float64 value of the nearest E4M3FN number (RNE, satfinite)."""
    return round_to_grid(x, mbits=3, emin=-6, maxval=E4M3_MAX, saturate=True)


def bf16_round(x):
    """float64 -> float64 value of the nearest bf16 (RNE, overflow to inf)."""
    return round_to_grid(x, mbits=7, emin=-126, maxval=BF16_MAX, saturate=False)


def bf16_bits(x):
    """float64 -> bf16 bit patterns (uint16) after RNE rounding."""
    r = bf16_round(x).astype(np.float32)  # exact: bf16 values are float32 values
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def fp32_round(x):
    """float64 -> float64 value of the nearest float32 (RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def floor_log2(a):
    """floor(log2 a) for finite a > 0 (float64), exact."""
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1
