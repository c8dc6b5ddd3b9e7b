"""Mutation tests of the oracle: every deliberate mistake must fail a pin.

[GAUDI] "Correctness" validates its converter the same way (seven deliberate
mutations of the tool, each caught by at least one encoding test).  Here each
mutant patches one piece of the oracle, then every argument-free pin test of
the oracle suite runs; at least one must fail.
"""

import inspect

import numpy as np
import pytest

import oracle.convert as OC
import oracle.formats as OF
import oracle.gemm as OG
import oracle.layer as OL
import oracle.permute as OP
import oracle.quant as OQ
import oracle.route as OR

from . import (test_oracle_convert, test_oracle_formats, test_oracle_gemm,
               test_oracle_quant, test_oracle_route_permute)

_orig_unpack = OF.unpack_fp4
_orig_e2m1 = OF.e2m1_decode
_orig_floor = OF.floor_log2
_orig_round = OF.round_to_grid
_orig_silu = OG.silu_mul
_orig_act = OL.activation_values
_orig_fp8q = OQ.fp8_quant_per_token
_orig_sigmoid = OR.sigmoid_fp32
_orig_route_token = OR.route_token
_orig_e4m3 = OF.e4m3_decode
_orig_mxdq = OF.mxfp4_dequant
_orig_nvdq = OF.nvfp4_dequant
_orig_combine = OG.moe_combine
_orig_permute = OP.moe_permute
_orig_nvqdq = OQ.nvfp4_qdq
_orig_e2m1_enc = OF.e2m1_encode
_orig_convert_row = OC.convert_row


def _fp8_scale_per_tensor(x_bits):
    """The per-token FP8 rule with one scale for the whole tensor."""
    codes, s = _orig_fp8q(x_bits)
    x = OF.bf16_decode(x_bits).astype(np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    st = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = (x / st).astype(np.float32)
    return OF.e4m3_encode(q.astype(np.float64)), np.full(x.shape[0], st, np.float32)


def _nvfp4_scale_per_row(afmt, x_bits):
    if afmt != "nvfp4" or x_bits.shape[0] == 0:
        return _orig_act(afmt, x_bits)
    return np.concatenate([_orig_act(afmt, x_bits[r:r + 1]) for r in range(x_bits.shape[0])])


def _swap_nibbles(packed):
    u = _orig_unpack(packed)
    out = u.copy()
    out[..., 0::2], out[..., 1::2] = u[..., 1::2], u[..., 0::2]
    return out


def _round_ties_away(x, mbits, emin, maxval, saturate):
    r = _orig_round(x, mbits, emin, maxval, saturate)
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, e - mbits)
    tie = (a / q) % 1 == 0.5
    up = np.copysign(np.minimum((np.floor(a / q) + 1) * q, maxval if saturate else np.inf), x)
    return np.where(tie, up, r)


def _combine_without_shared(y_sorted, pair_pos, topk_w, T, topk, n_shared):
    pos = np.asarray(pair_pos).reshape(T, topk + n_shared).copy()
    pos[:, topk:] = -1
    return _orig_combine(y_sorted, pos.reshape(-1), topk_w, T, topk, n_shared)


def _combine_shared_weighted(y_sorted, pair_pos, topk_w, T, topk, n_shared):
    """The shared slot scaled by the first routing weight instead of 1."""
    out, _ = _orig_combine(y_sorted, pair_pos, topk_w, T, topk, n_shared)
    pos = np.asarray(pair_pos).reshape(T, topk + n_shared)
    w = np.asarray(topk_w, dtype=np.float64).reshape(T, topk)
    for t in range(T):
        for i in range(n_shared):
            p = pos[t, topk + i]
            if p >= 0:
                out[t] += (w[t, 0] - 1.0) * y_sorted[p]
    return out, OF.bf16_bits(out)


def _permute_unstable(topk_ids, E, n_shared, block_m):
    """Pairs of one expert in descending pair order."""
    r = _orig_permute(topk_ids, E, n_shared, block_m)
    sp = r["sorted_pairs"].copy()
    offs = r["expert_offsets"]
    for e in range(len(offs) - 1):
        sp[offs[e]:offs[e + 1]] = sp[offs[e]:offs[e + 1]][::-1]
    pp = np.full_like(r["pair_pos"], -1)
    for i, q in enumerate(sp):
        if q >= 0:
            pp[q] = i
    return dict(r, sorted_pairs=sp, pair_pos=pp)


def _permute_tiles_unpadded(topk_ids, E, n_shared, block_m):
    """Tiles cut from all sorted rows at once, not per expert."""
    r = _orig_permute(topk_ids, E, n_shared, block_m)
    n = int(r["expert_offsets"][-1])
    offs = r["expert_offsets"]
    tiles = []
    for t0 in range(0, n, block_m):
        e = int(np.searchsorted(offs, t0, side="right") - 1)
        tiles.append((e, (t0 - int(offs[e])) // block_m))
    tiles = np.array(tiles, dtype=np.int32).reshape(-1, 2)
    return dict(r, tiles=tiles, n_tiles=len(tiles))


def _route_top1_group_score(logit_row, bias, n_group, topk_group, topk, renormalize=True,
                            routed_scale=1.0):
    """Groups ranked by their single largest key."""
    E = len(logit_row)
    s = OR.sigmoid_fp32(logit_row)
    key = (s + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    allowed = np.ones(E, dtype=bool)
    if n_group > 1:
        G = E // n_group
        gscore = np.array([key[g * G:(g + 1) * G].max() for g in range(n_group)], np.float32)
        allowed[:] = False
        for g in OR._order_desc(gscore)[:topk_group]:
            allowed[g * G:(g + 1) * G] = True
    cand = np.nonzero(allowed)[0]
    ids = cand[OR._order_desc(key[cand])][:topk].astype(np.int32)
    sel = s[ids].astype(np.float64)
    w = sel / sel.sum() if renormalize else sel.copy()
    return ids, w * float(routed_scale)


def _nvfp4_scale_without_6(x_bits, tensor_scale_in=None):
    """The dynamic NVFP4 tensor scale amax / 448 (the E2M1 maximum left out)."""
    if tensor_scale_in is None:
        x = OF.bf16_decode(x_bits).astype(np.float32)
        amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
        tensor_scale_in = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    return _orig_nvqdq(x_bits, tensor_scale_in)


def _grid_toward_zero(x, mbits, emin, maxval, saturate):
    """Rounding onto the grid by truncation instead of to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, e - mbits)
    r = np.where(a == 0, 0.0, np.floor(a / q) * q)
    r = np.where(r > maxval, maxval if saturate else np.inf, r)
    return np.copysign(r, x)


def _e2m1_saturate_at_4(x):
    return _orig_e2m1_enc(np.clip(np.asarray(x, dtype=np.float64), -4.0, 4.0))


def _convert_nan_blocks_in_max(codes_packed, scales):
    """Blocks with scale 255 taken into e_max as if their scale were 254."""
    s = np.asarray(scales).copy()
    fp8, k, status, inexact = _orig_convert_row(codes_packed, np.where(s == 255, 254, s))
    nan_blk = np.repeat(s == 255, 32)
    fp8 = np.where(nan_blk, np.uint8(0x7F), fp8).astype(np.uint8)
    return fp8, k, (2 if (s == 255).any() else status), inexact


def _route_unscaled(logit_row, bias, n_group, topk_group, topk, renormalize=True,
                    routed_scale=1.0):
    return _orig_route_token(logit_row, bias, n_group, topk_group, topk, renormalize, 1.0)


def _order_desc_high_first(values):
    idx = np.arange(len(values))
    return np.lexsort((-idx, -values.astype(np.float64)))


MUTANTS = {
    "k = e_max - 6": [(OC, "TOP_EXPONENT", 6)],
    "k = e_max - 8": [(OC, "TOP_EXPONENT", 8)],
    "nibble order swapped": [(OF, "unpack_fp4", _swap_nibbles)],
    "E2M1 sign dropped": [(OF, "e2m1_decode", lambda c: np.abs(_orig_e2m1(c)))],
    "E8M0 bias 128": [(OF, "e8m0_decode", lambda s: np.where(
        np.asarray(s) == 255, np.nan, np.ldexp(1.0, np.asarray(s, dtype=np.int64) - 128)))],
    "floor(log2) off by one": [(OF, "floor_log2", lambda a: _orig_floor(a) + 1)],
    "E8M0 255 not NaN": [(OF, "e8m0_decode", lambda s: np.ldexp(
        1.0, np.asarray(s, dtype=np.int64) - 127))],
    "RNE ties away from zero": [(OF, "round_to_grid", _round_ties_away)],
    "MX scale uses emax 1": [(OQ, "E2M1_EMAX", 1)],
    "routing ties to higher id": [(OR, "_order_desc", _order_desc_high_first)],
    "h not re-quantized before stage 2": [(OL, "stage2_activation",
                                           lambda afmt, h, h_bits, rounding=True:
                                           OF.bf16_decode(h_bits) if rounding else h)],
    "NVFP4 tensor scale per row": [(OL, "activation_values", _nvfp4_scale_per_row)],
    "FP8 activation scale per tensor, not per token": [(OQ, "fp8_quant_per_token",
                                                        _fp8_scale_per_tensor)],
    "gate/up swapped": [(OG, "silu_mul", lambda gu, I: _orig_silu(
        np.concatenate([gu[:, I:], gu[:, :I]], axis=1), I))],
    "sigmoid of +logit": [(OR, "sigmoid_fp32",
                           lambda l: _orig_sigmoid(-np.asarray(l, dtype=np.float32)))],
    "group score = largest key only": [(OR, "route_token", _route_top1_group_score)],
    "routed_scale ignored": [(OR, "route_token", _route_unscaled)],
    "E4M3 bias 8": [(OF, "e4m3_decode", lambda c: _orig_e4m3(c) * 0.5)],
    "NVFP4 tensor scale ignored": [(OF, "nvfp4_dequant", lambda p, s, ts: _orig_nvdq(p, s, 1.0))],
    "MX scale of the neighbouring block": [(OF, "mxfp4_dequant", lambda p, s: _orig_mxdq(
        p, np.roll(np.asarray(s), 1, axis=-1)))],
    "E2M1 code 7 is 5.0": [(OF, "E2M1_MAGNITUDES",
                            np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0]))],
    "SiLU sign flipped": [(OG, "silu_mul", lambda gu, I: gu[:, :I] / (1.0 + np.exp(
        np.clip(gu[:, :I], -700, 700))) * gu[:, I:])],
    "combine drops the shared expert": [(OG, "moe_combine", _combine_without_shared)],
    "combine weights the shared expert": [(OG, "moe_combine", _combine_shared_weighted)],
    "permutation unstable inside an expert": [(OP, "moe_permute", _permute_unstable)],
    "tiles not padded per expert": [(OP, "moe_permute", _permute_tiles_unpadded)],
    "NVFP4 tensor scale amax / 448": [(OQ, "nvfp4_qdq", _nvfp4_scale_without_6)],
    "rounding toward zero on every grid": [(OF, "round_to_grid", _grid_toward_zero)],
    "E2M1 encode saturates at 4": [(OF, "e2m1_encode", _e2m1_saturate_at_4)],
    "FP8 per-token scale amax / 240": [(OQ, "FP8_MAX", 240.0)],
    "E4M3 subnormal quantum 2^-10": [(OF, "e4m3_decode", lambda c: np.where(
        ((np.asarray(c, dtype=np.int64) >> 3) & 0xF) == 0, 0.5, 1.0) * _orig_e4m3(c))],
    "NaN blocks counted in the row maximum": [(OC, "convert_row", _convert_nan_blocks_in_max)],
}

PIN_MODULES = [test_oracle_formats, test_oracle_convert, test_oracle_quant,
               test_oracle_route_permute, test_oracle_gemm]


def _pin_tests():
    out = []
    for m in PIN_MODULES:
        for name, fn in sorted(vars(m).items()):
            if name.startswith("test_") and callable(fn) and not inspect.signature(fn).parameters:
                out.append((f"{m.__name__}.{name}", fn))
    return out


def test_pins_pass_unmutated():
    for name, fn in _pin_tests():
        fn()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_killed(mutant, monkeypatch):
    for mod, attr, val in MUTANTS[mutant]:
        monkeypatch.setattr(mod, attr, val)
    killed = []
    for name, fn in _pin_tests():
        try:
            with np.errstate(all="ignore"):
                fn()
        except AssertionError:
            # a failed check; an error raised by the mutant itself does not count
            killed.append(name)
        except Exception:
            pass
    assert killed, f"mutant '{mutant}' survived every pin"
