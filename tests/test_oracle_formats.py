"""Pins of oracle/formats.py against hand-worked values, brute force and library casts."""

import itertools
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_decodes():
    rows = []
    with open(os.path.join(GOLDEN, "fp4_decodes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, s, v0, v1 = line.split()
            rows.append((int(b, 16), int(s), float(v0), float(v1)))
    return rows


def test_hand_worked_decodes():
    rows = _golden_decodes()
    assert len(rows) >= 10
    for b, s, v0, v1 in rows:
        packed = np.zeros((1, 16), dtype=np.uint8)
        packed[0, 0] = b
        vals = F.mxfp4_dequant(packed, np.array([[s]], dtype=np.uint8))[0]
        assert vals[0] == v0 and np.signbit(vals[0]) == np.signbit(v0), (hex(b), s)
        assert vals[1] == v1 and np.signbit(vals[1]) == np.signbit(v1), (hex(b), s)
        assert np.all(vals[2:] == 0)


def test_e8m0_special_codes():
    v = F.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126
    assert v[2] == 0.5 and v[3] == 1.0 and v[4] == 2.0
    assert v[5] == 2.0 ** 127 and np.isnan(v[6])


def test_pack_unpack_roundtrip_and_order():
    codes = np.arange(32, dtype=np.uint8) % 16
    p = F.pack_fp4(codes)
    assert p[0] == 0x10 and p[1] == 0x32  # element 0 low nibble, element 1 high nibble
    assert np.array_equal(F.unpack_fp4(p), codes)
    g = np.random.default_rng(0).integers(0, 256, size=(5, 64), dtype=np.uint8)
    assert np.array_equal(F.pack_fp4(F.unpack_fp4(g)), g)


def test_mxfp4_bytes_per_value():
    # [ATOM] "MXFP4 Tensor Anatomy": 16 B payload + 1 B scale per 32 values.
    K = 7168
    assert (K // 2 + K // 32) / K == 0.53125


def _brute_nearest_even(x, grid_vals, grid_codes, even_key):
    """Nearest grid value; ties broken toward the code whose even_key is even."""
    d = np.abs(grid_vals - x)
    best = d.min()
    cands = [i for i in range(len(grid_vals)) if d[i] == best]
    if len(cands) > 1:
        cands = [i for i in cands if even_key(grid_codes[i]) % 2 == 0]
    assert len(cands) == 1, (x, cands)
    return grid_codes[cands[0]]


def test_e2m1_encode_brute_force():
    # grid: the 8 non-negative E2M1 values; ties to even significand (code LSB)
    codes = np.arange(8)
    vals = F.E2M1_MAGNITUDES
    xs = list(np.linspace(0, 7.5, 301)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0]
    for x in xs:
        c = int(F.e2m1_encode(np.array([x]))[0])
        if x > 6:
            assert c == 7
            continue
        assert c == _brute_nearest_even(x, vals, codes, lambda c: c), x
        cn = int(F.e2m1_encode(np.array([-x]))[0])
        assert cn == c | 8
    # explicit ties
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in ties.items():
        assert int(F.e2m1_encode(np.array([x]))[0]) == c


def test_e2m1_decode_all_codes():
    v = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(v[:8]) == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert list(-v[8:]) == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(v[8])


def test_e4m3_decode_matches_torch():
    allc = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allc).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mine = F.e4m3_decode(allc)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan].astype(np.float64), mine[~nan])
    assert F.e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_encode_brute_force():
    finite = np.array([c for c in range(128) if c != 0x7F])
    vals = F.e4m3_decode(finite)
    g = np.random.default_rng(1)
    xs = np.concatenate([vals, (vals[1:] + vals[:-1]) / 2,       # every tie point
                         g.uniform(0, 460, 2000), g.uniform(0, 2 ** -5, 2000)])
    enc = F.e4m3_encode(xs)
    for x, c in zip(xs, enc):
        if x > 448:
            assert c == 0x7E
            continue
        assert c == _brute_nearest_even(x, vals, finite, lambda c: c), x
    assert np.array_equal(F.e4m3_encode(-xs[xs <= 448]), enc[xs <= 448] | 0x80)


def test_e4m3_encode_matches_torch_cast():
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(20000) * 30, g.standard_normal(2000) * 1e-3])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x.astype(np.float64)), ref)


def test_bf16_round_matches_torch():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(50000) * 100, g.standard_normal(1000) * 1e-39,
                        g.standard_normal(1000) * 1e37]).astype(np.float32)
    # add exact ties: bf16 values plus half an ulp
    b = torch.from_numpy(x[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    tie = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, tie])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_bits(x.astype(np.float64)), ref)
    assert np.array_equal(F.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def test_fp32_grid_matches_numpy_cast():
    g = np.random.default_rng(4)
    x = g.standard_normal(20000) * np.exp(g.uniform(-80, 80, 20000))
    r = F.round_to_grid(x, mbits=23, emin=-126, maxval=float(np.finfo(np.float32).max),
                        saturate=False)
    assert np.array_equal(r, x.astype(np.float32).astype(np.float64))


def test_floor_log2():
    for e in range(-140, 130):
        for m in (1.0, 1.5, 1.999):
            assert F.floor_log2(np.ldexp(m, e)) == e


def test_nvfp4_dequant_small():
    packed = F.pack_fp4(np.array([[7, 15] + [0] * 14], dtype=np.uint8))
    sc = F.e4m3_encode(np.array([[1.5]]))
    v = F.nvfp4_dequant(packed, sc, 0.25)
    assert v[0, 0] == 6 * 1.5 * 0.25 and v[0, 1] == -6 * 1.5 * 0.25


@pytest.mark.parametrize("c", list(itertools.product(range(16), repeat=2))[:40])
def test_unpack_each_byte(c):
    lo, hi = c
    p = np.array([lo | (hi << 4)], dtype=np.uint8)
    assert list(F.unpack_fp4(p)) == [lo, hi]
