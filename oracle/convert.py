"""Exact MXFP4 -> FP8 E4M3 per-channel conversion.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GAUDI] "Exact MXFP4 to FP8 per-channel conversion".  Per output row
(channel) x of decoded values:
    e_max = exponent of max_i |x_i|,   k = e_max - 7,   scale = 2^k,
    code_i = E4M3(x_i / 2^k).
The page's claim, restated: if the row's E8M0 scales lie within 9
consecutive binades, every x_i / 2^k is zero or an E4M3 normal with exponent
in [-5, 7] and magnitude <= 192 = 1.5 * 2^7, so decode(code_i) * 2^k == x_i.

Readings for what the page leaves open:
  * "exponent of the largest element" = floor(log2 max |x|) over the row's
    decoded values (blocks with scale 255 excluded).
  * Each element is encoded by E4M3 round-to-nearest-even with OCP E4M3FN
    subnormals; for rows inside the 9-binade bound this is exact.
  * row_status: 0 every element exact with exponent in [-5, 7];
    1 some non-zero element has an exponent below the -5 floor (the page's
    bound is exceeded; the code may or may not still be exact);
    2 a block of the row has E8M0 code 255 (NaN): those elements get code
    0x7F and k comes from the finite blocks; 3 the finite part of the row is
    all zero: k = 0, channel scale 1.0.  Precedence 2 > 3 > 1 > 0.
  * inexact[row] is True when some finite element differs from
    decode(code) * 2^k.
"""

import numpy as np

from . import formats as F

TOP_EXPONENT = 7     # E4M3 exponent given to the row's largest element
FLOOR_EXPONENT = -5  # lowest element exponent the page's guarantee covers


def convert_row(codes_packed, scales):
    """One row: packed E2M1 [K/2], E8M0 [K/32] -> (fp8 [K], scale_f32, status, inexact)."""
    x = F.mxfp4_dequant(codes_packed[None], scales[None])[0]
    nan_blk = np.repeat(np.asarray(scales) == 255, 32)
    fin = ~nan_blk
    nz = fin & (x != 0)
    if nz.any():
        e_max = int(F.floor_log2(np.abs(x[nz]).max()))
        k = e_max - TOP_EXPONENT
        zero_row = False
    else:
        k = 0
        zero_row = True
    scaled = np.where(fin, x, 0.0) / np.ldexp(1.0, k)          # exact
    codes = F.e4m3_encode(scaled)
    codes = np.where(nan_blk, np.uint8(0x7F), codes).astype(np.uint8)
    back = F.e4m3_decode(np.where(nan_blk, 0, codes)) * np.ldexp(1.0, k)
    inexact = bool(np.any(back[fin] != x[fin]))
    below = bool(nz.any() and (F.floor_log2(np.abs(scaled[nz])).min() < FLOOR_EXPONENT))
    if nan_blk.any():
        status = 2
    elif zero_row:
        status = 3
    elif below:
        status = 1
    else:
        status = 0
    return codes, np.float32(np.ldexp(1.0, k)), status, inexact


def mxfp4_to_fp8_channel(codes, scales):
    """codes uint8 [R, K/2], scales uint8 [R, K/32] -> dict(fp8, scale, status, n_inexact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R = codes.shape[0]
    K = codes.shape[1] * 2
    fp8 = np.empty((R, K), dtype=np.uint8)
    sc = np.empty(R, dtype=np.float32)
    st = np.empty(R, dtype=np.uint8)
    n_inexact = 0
    for r in range(R):
        fp8[r], sc[r], st[r], inex = convert_row(codes[r], scales[r])
        n_inexact += int(inex)
    return dict(fp8=fp8, scale=sc, status=st, n_inexact=n_inexact)
