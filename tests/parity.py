"""Comparison helpers of the parity tests (bit-exact and float tolerances).

Float outputs of the HIP path (bf16) are compared with the oracle's value
rounded to bf16 at the same rounding points:
  rel-L2 = ||gpu - ref|| / ||ref|| <= 1e-3, and
  |gpu - ref| <= max(1e-2 * RMS(ref), one bf16 ulp of ref) element-wise.
The ulp allowance admits rounding-boundary flips caused by a different (but
valid) float32 accumulation order; flips are counted and reported.
"""

import numpy as np

from oracle import formats as F

REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2


def bf16_ulp(r):
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.where(a > 0, np.floor(np.log2(np.maximum(a, 1e-300))), -133)
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))


def assert_float_close(gpu, ref, name, rel_l2=REL_L2, max_abs_rms=MAX_ABS_RMS):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    if r.size == 0:
        return {}
    d = np.abs(g - r)
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nr if nr > 0 else np.linalg.norm(g - r)
    rms = np.sqrt(np.mean(r * r))
    allow = np.maximum(max_abs_rms * rms, bf16_ulp(r))
    bad = d > allow
    stats = dict(rel_l2=float(rel), max_abs=float(d.max()), rms=float(rms),
                 flips=int(np.count_nonzero(d > 0)), n=int(r.size))
    assert rel <= rel_l2, f"{name}: rel-L2 {rel:.3e} > {rel_l2} ({stats})"
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements beyond max(1e-2*RMS, 1 ulp); "
                           f"worst {d.max():.4g} ({stats})")
    return stats


def assert_bf16_close(gpu_bits, ref_vals, name):
    """gpu_bits: bf16 bit patterns; ref_vals: oracle values (rounded to bf16 here)."""
    return assert_float_close(F.bf16_decode(np.asarray(gpu_bits).view(np.uint16)),
                              F.bf16_round(ref_vals), name)


def assert_equal(gpu, ref, name):
    g, r = np.asarray(gpu), np.asarray(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    if not np.array_equal(g, r):
        idx = np.argwhere(g != r)
        raise AssertionError(f"{name}: {len(idx)} mismatches, first at {idx[0].tolist()}: "
                             f"gpu={g[tuple(idx[0])]} ref={r[tuple(idx[0])]}")
