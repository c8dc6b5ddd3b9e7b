"""Pins of oracle/quant.py: the MXFP4 scale rule, brute-force codes, NVFP4 round trips."""

import numpy as np
import torch

from oracle import formats as F
from oracle import quant as Q


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _nearest_e2m1_code(q):
    """Brute force over the 16 codes: nearest value, ties to the even code, sign kept."""
    mags = F.E2M1_MAGNITUDES
    a = min(abs(q), 6.0)
    d = np.abs(mags - a)
    c = [i for i in range(8) if d[i] == d.min()]
    if len(c) > 1:
        c = [i for i in c if i % 2 == 0]
    return c[0] | (8 if np.signbit(q) else 0)


def test_mxfp4_scale_rule_and_codes_brute_force():
    g = np.random.default_rng(20)
    x = g.standard_normal((7, 96)) * np.exp(g.uniform(-6, 6, (7, 1)))
    xb = _bf16(x)
    codes, scales = Q.mxfp4_quant_1x32(xb)
    xv = F.bf16_decode(xb)
    c = F.unpack_fp4(codes)
    for r in range(7):
        for b in range(3):
            blk = xv[r, 32 * b:32 * b + 32]
            e = int(scales[r, b]) - 127
            amax = np.abs(blk).max()
            assert 4 <= amax / 2.0 ** e < 8          # largest element maps into [4, 8)
            for i in range(32):
                assert c[r, 32 * b + i] == _nearest_e2m1_code(blk[i] / 2.0 ** e)


def test_mxfp4_hand_examples():
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, :6] = [6.0, -3.0, 0.25, 0.75, -0.1, 5.0]
    codes, scales = Q.mxfp4_quant_1x32(_bf16(blk))
    assert scales[0, 0] == 127                        # floor(log2 6) - 2 = 0
    c = F.unpack_fp4(codes)[0]
    assert list(c[:6]) == [7, 8 | 5, 0, 2, 8 | 0, 6]  # 0.25 -> 0, 0.75 -> 1.0, 5 -> 4
    blk2 = np.full((1, 32), 1.0, dtype=np.float32)
    codes, scales = Q.mxfp4_quant_1x32(_bf16(blk2))
    assert scales[0, 0] == 125 and np.all(F.unpack_fp4(codes) == 6)   # 1.0 = 4 * 2^-2


def test_mxfp4_zero_and_tiny_blocks():
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :32] = -0.0
    x[1, 32] = 2.0 ** -130        # bf16 subnormal: scale clamps at code 0 (2^-127)
    x[1, 33] = -(2.0 ** -133)
    codes, scales = Q.mxfp4_quant_1x32(_bf16(x))
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 1] == 0
    c = F.unpack_fp4(codes)
    assert np.all(c[0, :32] == 8)  # -0.0 keeps its sign
    assert c[1, 32] == 0           # 2^-130 / 2^-127 = 0.125 -> 0
    assert c[1, 33] == 8


def test_mxfp4_error_bound():
    g = np.random.default_rng(21)
    xb = _bf16(g.standard_normal((16, 256)))
    codes, scales = Q.mxfp4_quant_1x32(xb)
    x = F.bf16_decode(xb)
    d = F.mxfp4_dequant(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    # |x - q| <= half a quantum, where the quantum at magnitude a is 2^(floor(log2 a)-1)
    q = np.abs(x) / 2.0 ** e
    quantum = np.where(q < 1, 0.5, 2.0 ** (np.floor(np.log2(np.maximum(q, 1))) - 1)) * 2.0 ** e
    # the floor-based scale maps the block max into [4, 8); magnitudes above 6 saturate
    bound = np.maximum(quantum / 2, (q - 6) * 2.0 ** e)
    assert np.all(np.abs(x - d) <= bound + 1e-300)
    assert np.any(q > 6)   # the sample does exercise saturation


def test_nvfp4_on_grid_roundtrip_static_scale():
    g = np.random.default_rng(22)
    M, K = 4, 64
    st = 0.5
    codes = g.integers(0, 16, (M, K)).astype(np.uint8)
    sb = F.e4m3_decode(g.integers(0x30, 0x50, (M, K // 16)))     # moderate E4M3 scales
    codes.reshape(M, K // 16, 16)[..., 0] = 7                      # block amax = 6
    x = F.e2m1_decode(codes) * np.repeat(sb, 16, axis=1) * st
    xb = F.bf16_bits(x)
    assert np.array_equal(F.bf16_decode(xb), x)                    # x is bf16-exact
    r = Q.nvfp4_qdq(xb, tensor_scale_in=st)
    assert np.array_equal(r["y"], xb)
    assert np.array_equal(F.e4m3_decode(r["scales"]), sb)
    nz = F.e2m1_decode(codes) != 0
    assert np.array_equal(F.unpack_fp4(r["codes"])[nz], codes[nz])


def test_nvfp4_codes_brute_force_dynamic():
    g = np.random.default_rng(23)
    xb = _bf16(g.standard_normal((8, 128)) * 3)
    r = Q.nvfp4_qdq(xb)
    x = F.bf16_decode(xb).astype(np.float32)
    st = np.float32(np.float32(np.abs(x).max()) / np.float32(2688))
    assert r["tensor_scale"] == st
    sb = F.e4m3_decode(r["scales"])
    c = F.unpack_fp4(r["codes"])
    for i in range(8):
        for b in range(8):
            blk = x[i, 16 * b:16 * b + 16]
            want_sb = F.e4m3_round(np.float64(np.float32(np.abs(blk).max() / np.float32(6 * st))))
            assert sb[i, b] == want_sb
            d = np.float32(np.float32(sb[i, b]) * st)
            for j in range(16):
                q = np.float32(blk[j] / d)
                assert c[i, 16 * b + j] == _nearest_e2m1_code(float(q))
    y = F.bf16_decode(r["y"])
    # the round trip stays within half an E2M1 step of the block scale
    err = np.abs(y - F.bf16_decode(xb))
    assert np.all(err <= np.repeat(sb * st, 16, axis=1) * 1.0 + 1e-30)


def test_nvfp4_zero_tensor():
    r = Q.nvfp4_qdq(np.zeros((2, 32), dtype=np.uint16))
    assert r["tensor_scale"] == 1.0 and np.all(r["y"] == 0) and np.all(r["scales"] == 0)


# --------------------------------------------------------------------------
# Dynamic per-token FP8 (the W8A8 activations)
# --------------------------------------------------------------------------

def _e4m3_table():
    """Every finite OCP E4M3FN code and its value, from the bit fields."""
    out = []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        e, m = (c >> 3) & 15, c & 7
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        out.append((c, -v if c & 0x80 else v))
    return out


def _nearest_e4m3_code(q):
    """Brute force: nearest finite value (saturating), ties to the even mantissa, sign kept."""
    tab = [(c, v) for c, v in _e4m3_table() if (c & 0x80) == (0x80 if np.signbit(q) else 0)]
    a = min(abs(q), 448.0)
    d = [abs(abs(v) - a) for _, v in tab]
    best = [c for (c, _), di in zip(tab, d) if di == min(d)]
    if len(best) > 1:
        best = [c for c in best if c % 2 == 0]
    return best[0]


def test_fp8_per_token_scale_and_codes_brute_force():
    g = np.random.default_rng(21)
    x = g.standard_normal((6, 40)) * np.exp(g.uniform(-8, 8, (6, 1)))
    x[2, 5] = 0.0
    xb = _bf16(x)
    codes, s = Q.fp8_quant_per_token(xb)
    xv = F.bf16_decode(xb).astype(np.float32)
    for r in range(6):
        amax = np.float32(np.abs(xv[r]).max())
        assert s[r] == np.float32(amax / np.float32(448.0))
        for i in range(40):
            q = float(np.float32(xv[r, i] / s[r]))
            assert codes[r, i] == _nearest_e4m3_code(q), (r, i, q)
        # the row maximum lands on +-448
        i = int(np.argmax(np.abs(xv[r])))
        assert codes[r, i] & 0x7F == 0x7E


def test_fp8_per_token_hand_example_and_zero_row():
    xb = _bf16([[1.0, -2.0, 0.5, 0.0], [0.0, -0.0, 0.0, 0.0]])
    codes, s = Q.fp8_quant_per_token(xb)
    assert s[0] == np.float32(np.float32(2.0) / np.float32(448.0)) and s[1] == 1.0
    # 1 / s = 224 = 1.75 * 2^7, 2 / s = 448, 0.5 / s = 112 = 1.75 * 2^6
    assert codes[0].tolist() == [0x76, 0xFE, 0x6E, 0x00]
    assert codes[1].tolist() == [0x00, 0x80, 0x00, 0x00]
    v = Q.fp8_qdq_values(xb)
    assert v[0, 1] == -448.0 * float(s[0]) and v[1].tolist() == [0.0, -0.0, 0.0, 0.0]
