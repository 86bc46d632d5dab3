"""Pins of the oracle's K quantizer (thumbnail + residual) against exact arithmetic.

The page ("Faster Than Flash", Method section 1) fixes only that K is split
into a 2-bit thumbnail and an 8-bit residual; the convention itself is the
repository's.  These tests check ``oracle.ffd_oracle.quantize_k`` against an
exact-rational brute force, closed-form error bounds and special cases.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import ffd_oracle as orc


def _f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


# ---------------------------------------------------------------- rounding
def test_rne_binary16_matches_hand_examples():
    # 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10: ties to even -> 1
    assert bf.rne_binary16(Fraction(1) + Fraction(1, 2 ** 11)) == 1
    # 1 + 3*2^-11 is the midpoint between 1+2^-10 and 1+2^-9: ties to even -> 1+2^-9
    assert bf.rne_binary16(Fraction(1) + Fraction(3, 2 ** 11)) == 1 + Fraction(1, 2 ** 9)
    # smallest subnormal 2^-24; half of it ties to 0 (even)
    assert bf.rne_binary16(Fraction(1, 2 ** 24)) == Fraction(1, 2 ** 24)
    assert bf.rne_binary16(Fraction(1, 2 ** 25)) == 0
    assert bf.rne_binary16(Fraction(3, 2 ** 25)) == Fraction(2, 2 ** 24)
    assert bf.rne_binary16(Fraction(65504)) == 65504
    assert bf.rne_binary16(Fraction(1, 3)) == Fraction(1365, 4096)   # 0x3555


def test_f16_round_is_correctly_rounded_from_fp64():
    """numpy's float64 -> float16 cast (used by the oracle) equals exact RNE."""
    rng = np.random.default_rng(0)
    mags = np.concatenate([
        rng.uniform(0, 1, 3000) * 2.0 ** rng.integers(-30, 16, 3000),
        rng.uniform(0, 1, 1000) * 2.0 ** -24,
    ])
    # exact midpoints between neighbouring fp16 values (ties)
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16).view(np.float16).astype(np.float64)
    h2 = (rng.integers(0, 0x7BFF, 2000).astype(np.uint16) + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    lo = np.minimum(h, h2)
    nxt = np.nextafter(lo.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mids = (lo + nxt) / 2
    xs = np.concatenate([mags, -mags[:500], mids])
    got = orc.f16_round(xs)
    for x, g in zip(xs, got):
        assert Fraction(float(g)) == bf.rne_binary16(Fraction(float(x))), x


# ---------------------------------------------------------------- quantizer vs brute force
def _groups_zoo(rng):
    out = []
    out.append(rng.standard_normal(128))                              # plain
    x = rng.standard_normal(128); x[[3, 40, 77, 120]] *= 5; out.append(x)   # outlier channels
    out.append(np.full(128, 0.75))                                      # constant groups
    out.append(np.zeros(128))                                           # all zero
    out.append(rng.standard_normal(128) * 2.0 ** -20)                   # subnormal-scale values
    out.append(rng.standard_normal(128) * 2.0 ** 12)                    # large values
    x = rng.standard_normal(128); x[::2] = 0; out.append(x)             # half zeros
    # on-grid group: values z + c*s with both extremes present
    c = rng.integers(0, 4, 128); c[0] = 0; c[1] = 3
    out.append(-1.5 + c * 0.25)
    # values sitting exactly on a code decision boundary (x - z = (k - 1/2) s)
    x = np.zeros(128); x[0] = 0.0; x[1] = 3.0; x[2:6] = [0.5, 1.5, 2.5, 1.0]; out.append(x)
    # residual ties: values whose residual hits (j - 1/2) * rscale
    x = rng.standard_normal(128); x[0] = x.min() - 1; out.append(x)
    # mixed magnitudes in one group
    x = rng.standard_normal(128) * 2.0 ** rng.integers(-14, 8, 128); out.append(x)
    return [_f16(v) for v in out]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_k_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(seed)
    toks = np.stack(_groups_zoo(rng) + [_f16(rng.standard_normal(128) * rng.uniform(0.01, 8)) for _ in range(20)])
    pk = orc.quantize_k(toks)
    deq2, khat = orc.dequantize(pk)
    for i, t in enumerate(toks):
        ref = bf.pack_token([float(v) for v in t])
        assert list(pk["codes"][i]) == ref["codes"], i
        assert list(pk["res"][i]) == ref["res"], i
        for g in range(4):
            assert Fraction(float(pk["scale"][i, g])) == ref["scale"][g]
            assert Fraction(float(pk["zero"][i, g])) == ref["zero"][g]
            assert Fraction(float(pk["rscale"][i, g])) == ref["rscale"][g]
        assert [Fraction(float(v)) for v in deq2[i]] == ref["deq2"]
        assert [Fraction(float(v)) for v in khat[i]] == ref["khat"]


def test_codes_and_residuals_in_range():
    rng = np.random.default_rng(5)
    K = _f16(rng.standard_normal((2000, 128)) * 3)
    pk = orc.quantize_k(K)
    assert pk["codes"].max() <= 3
    assert np.abs(pk["res"].astype(int)).max() <= 127
    assert (pk["scale"] >= 0).all() and (pk["rscale"] >= 0).all()


def test_error_bounds_closed_form():
    """|x - deq2| <= s/2 except the clamped top code, |x - K-hat| <= s8/2 (normal scales)."""
    rng = np.random.default_rng(7)
    K = _f16(rng.standard_normal((4000, 128)) * rng.uniform(0.05, 20, (4000, 1)))
    pk = orc.quantize_k(K)
    deq2, khat = orc.dequantize(pk)
    x = K.astype(np.float64).reshape(-1, 4, 32)
    d2 = np.abs(x - deq2.reshape(-1, 4, 32))
    s = pk["scale"].astype(np.float64)[..., None]
    s8 = pk["rscale"].astype(np.float64)[..., None]
    normal = (s >= 2.0 ** -14) & (s8 >= 2.0 ** -14)
    # clamped top code: s = RNE(range/3) may be below range/3 by <= 2^-11 relative
    bound2 = s / 2 + 3 * s * 2.0 ** -11
    assert (d2 <= bound2)[np.broadcast_to(normal, d2.shape)].all()
    d8 = np.abs(x - khat.reshape(-1, 4, 32))
    bound8 = s8 / 2 + 127 * s8 * 2.0 ** -11
    assert (d8 <= bound8)[np.broadcast_to(normal, d8.shape)].all()
    # residual rebuilds K far better than the thumbnail alone
    assert d8.max() < d2.max() / 20


def test_constant_and_on_grid_groups_are_exact():
    g = np.full(128, 1.25)
    c = np.arange(128) % 4
    grid = -0.5 + c * 0.125                      # z = -0.5, s = 0.125, extremes present
    K = _f16(np.stack([g, grid]))
    pk = orc.quantize_k(K)
    deq2, khat = orc.dequantize(pk)
    assert (pk["scale"][0] == 0).all() and (pk["codes"][0] == 0).all() and (pk["res"][0] == 0).all()
    assert (pk["scale"][1] == np.float16(0.125)).all()
    assert (pk["codes"][1] == c).all()
    assert (pk["res"][1] == 0).all() and (pk["rscale"][1] == 0).all()
    assert np.array_equal(khat, K.astype(np.float64))
    assert np.array_equal(deq2[1], K[1].astype(np.float64))


def test_signed_zero_minimum_is_stored_as_plus_zero():
    x = np.zeros((1, 128), np.float16)
    x[0, 5] = np.float16(-0.0)
    x[0, 40:72] = np.float16(-0.0)
    pk = orc.quantize_k(x)
    assert (pk["zero"].view(np.uint16) == 0).all()
    assert (pk["scale"].view(np.uint16) == 0).all() and (pk["rscale"].view(np.uint16) == 0).all()


def test_tiny_residual_below_rscale_resolution_is_dropped():
    """A residual too small for a nonzero fp16 rscale leaves res = 0 (rscale = 0)."""
    x = np.zeros(32)
    x[1] = 3 * 2.0 ** -14                     # scale = 2^-14, on grid
    x[2] = 2.0 ** -14 + 2.0 ** -24            # off grid by one subnormal ulp
    K = _f16(np.concatenate([x, np.zeros(96)]))[None]
    pk = orc.quantize_k(K)
    ref = bf.pack_group([float(v) for v in K[0, :32]])
    assert Fraction(float(pk["rscale"][0, 0])) == ref["rscale"]
    assert list(pk["res"][0, :32]) == ref["res"]
