"""Pins of oracle/convert.py (MXFP4 -> FP8 E4M3 per-channel).

Test list follows [GAUDI] "Correctness": adversarial rows, the -5 floor edge,
E8M0 0/254/255, the load-time halving replayed, element-exact validation; the
mutation tests live in test_oracle_mutants.py.
"""

import os

import numpy as np

import synth
from oracle import convert as C
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_convert_golden():
    cases = []
    with open(os.path.join(GOLDEN, "fp8_convert.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, sc, by, k, f8, st, inex = [s.strip() for s in line.split("|")]
            scales = np.array([int(v) for v in sc.split()], dtype=np.uint8)
            packed = np.zeros(32, dtype=np.uint8)
            for it in by.split():
                i, h = it.split(":")
                packed[int(i)] = int(h, 16)
            fp8 = np.zeros(64, dtype=np.uint8)
            for it in f8.split():
                i, h = it.split(":")
                if "-" in i:
                    a, b = i.split("-")
                    fp8[int(a):int(b) + 1] = int(h, 16)
                else:
                    fp8[int(i)] = int(h, 16)
            cases.append((name, packed, scales, int(k), fp8, int(st), int(inex)))
    return cases


def test_golden_conversions():
    cases = load_convert_golden()
    assert len(cases) == 7
    for name, packed, scales, k, fp8, st, inex in cases:
        codes, sc, status, inexact = C.convert_row(packed, scales)
        assert np.array_equal(codes, fp8), name
        assert sc == np.float32(2.0 ** k), name
        assert status == st and int(inexact) == inex, name


def test_exactness_invariant_span_le_9():
    R, K = 400, 256
    g = np.random.default_rng(40)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales, span = synth.spanned_scales(R, K // 32, 5, 99, span_lo=0, span_hi=9)
    res = C.mxfp4_to_fp8_channel(codes, scales)
    assert res["n_inexact"] == 0 and np.all(res["status"] == 0)
    x = F.mxfp4_dequant(codes, scales)
    back = F.e4m3_decode(res["fp8"]) * res["scale"].astype(np.float64)[:, None]
    assert np.array_equal(back, x)                 # element-exact
    # every non-zero code is an E4M3 normal with exponent in [-5, 7], magnitude <= 192
    nz = (res["fp8"] & 0x7F) != 0
    ef = (res["fp8"] >> 3) & 0xF
    assert np.all(ef[nz] >= 2) and np.all(ef[nz] <= 14)
    assert np.abs(F.e4m3_decode(res["fp8"])).max() <= 192
    # the row's largest element has exponent exactly 7
    assert np.all(ef.max(axis=1) == 14)


def test_spans_above_9_flagged():
    R, K = 300, 128
    g = np.random.default_rng(41)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    codes[:, :] |= 0x11        # no zero nibbles: every block has 0.5-or-larger elements
    scales, span = synth.spanned_scales(R, K // 32, 5, 98, span_lo=10, span_hi=16)
    res = C.mxfp4_to_fp8_channel(codes, scales)
    x = F.mxfp4_dequant(codes, scales)
    back = F.e4m3_decode(res["fp8"]) * res["scale"].astype(np.float64)[:, None]
    exact_rows = np.all(back == x, axis=1)
    assert res["n_inexact"] == int((~exact_rows).sum()) > 0
    assert np.all(res["status"][~exact_rows] == 1)


def test_halving_replayed_stays_normal():
    # [GAUDI]: the load-time halving of FP8 weights keeps every element normal
    # thanks to the -5 floor (exponent -6 is still an E4M3 normal).
    R, K = 200, 256
    g = np.random.default_rng(42)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales, _ = synth.spanned_scales(R, K // 32, 5, 97, span_lo=9, span_hi=9)
    res = C.mxfp4_to_fp8_channel(codes, scales)
    v = F.e4m3_decode(res["fp8"])
    half = v / 2
    enc = F.e4m3_encode(half)
    assert np.array_equal(F.e4m3_decode(enc), half)
    nz = half != 0
    assert np.all(((enc >> 3) & 0xF)[nz] >= 1)     # normal after halving


def test_extreme_scales_rows():
    g = np.random.default_rng(43)
    for top in (0, 9, 254):
        codes = g.integers(0, 256, (1, 64), dtype=np.uint8)
        scales = np.full((1, 4), top, dtype=np.uint8)
        res = C.mxfp4_to_fp8_channel(codes, scales)
        x = F.mxfp4_dequant(codes, scales)
        back = F.e4m3_decode(res["fp8"]) * np.float64(res["scale"][0])
        assert np.array_equal(back, x) and res["status"][0] == 0


def test_nan_scale_rows():
    codes = np.full((1, 64), 0x77, dtype=np.uint8)
    scales = np.array([[127, 255, 120, 255]], dtype=np.uint8)
    res = C.mxfp4_to_fp8_channel(codes, scales)
    assert res["status"][0] == 2
    assert np.all(res["fp8"][0, 32:64] == 0x7F) and np.all(res["fp8"][0, 96:128] == 0x7F)
    assert res["scale"][0] == np.float32(2.0 ** (2 - 7))
    assert np.all(res["fp8"][0, :32] == 0x74)
