"""Closed-form pin of the Top-delta rule on a hand-built cache (tests/golden/top_delta_closed_form.json).

Keys are placed on the quantizer's grid so estimated and exact scores are
known exactly; the expected pseudo-max, threshold and kept blocks are worked
out by hand from the page's criterion and stored in the fixture.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import ffd_oracle as orc

FIX = os.path.join(os.path.dirname(__file__), "golden", "top_delta_closed_form.json")


def build(fx):
    L = fx["L"]
    v = np.full(L, fx["default_score"])
    for t, s in fx["scores"].items():
        v[int(t)] = s
    K = np.zeros((L, 128))
    K[:, 0] = v
    K[:, 1:32] = (v - 0.75)[:, None]
    q = np.zeros((1, 128), np.float16)
    q[0, 0] = 1.0
    return q, K.astype(np.float16), v


def test_fixture_keys_are_exact_on_the_grid():
    fx = json.load(open(FIX))
    q, K, v = build(fx)
    pk = orc.quantize_k(K)
    deq2, khat = orc.dequantize(pk)
    np.testing.assert_array_equal(deq2, K.astype(np.float64))
    np.testing.assert_array_equal(khat, K.astype(np.float64))
    np.testing.assert_array_equal(orc.scores(q, khat, 1.0)[0], v)


@pytest.mark.parametrize("case", [0, 1])
def test_top_delta_closed_form(case):
    fx = json.load(open(FIX))
    c = fx["cases"][case]
    q, K, v = build(fx)
    V = np.random.default_rng(case).standard_normal((fx["L"], 128)).astype(np.float16)
    r = orc.decode_head(q, orc.quantize_k(K), V, fx["L"], c["delta"], 1.0, fx["sink"], fx["local"])
    assert r["m_tilde"][0] == c["m_tilde"]
    assert r["thr"][0] == c["threshold"]
    assert list(r["keep"]) == c["keep"]
    tok = np.nonzero(np.repeat(np.array(c["keep"]), 64)[: fx["L"]])[0]
    ref = softmax(v[tok]) @ V[tok].astype(np.float64)
    np.testing.assert_allclose(r["out"][0], ref, rtol=0, atol=1e-12)
    # the page's reading of delta: kept non-forced blocks reach weight e^-delta of the pseudo-max
    w = np.exp(r["bmax"][0] - r["m_tilde"][0])
    nf = ~r["forced"]
    assert (w[nf & r["keep"]] >= np.exp(-c["delta"])).all()
    assert (w[nf & ~r["keep"]] < np.exp(-c["delta"])).all()
