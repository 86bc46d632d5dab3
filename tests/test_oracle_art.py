"""Pins of the oracle's run-time termination of the refine stream (the ART
page, "Attention Run-time Termination", Method sections 2.2-2.4, applied to
each chunk's stream of kept blocks)."""
import math

import numpy as np
import pytest

from oracle import ffd_oracle as orc
from tests.test_oracle_decode import SCALE, _case


def test_chunk_blocks_partition_the_sequence():
    for nblk, cb, nchunk in [(64, 4, 16), (100, 16, 7), (5, 8, 1), (257, 3, 86), (1, 1, 1)]:
        nchunk = max(nchunk, math.ceil(nblk / cb))
        lists = orc.chunk_blocks(nblk, cb, nchunk)
        flat = sorted(b for l in lists for b in l)
        assert flat == list(range(nblk))
        assert all(len(l) <= cb and l == sorted(l) for l in lists)


def test_disabled_stop_is_plain_decode():
    L, G = 3000, 4
    q, K, V = _case(L, G, seed=51)
    pk = orc.quantize_k(K)
    ref = orc.decode_head(q, pk, V, L, 4.0, SCALE)
    got = orc.art_decode_head(q, pk, V, L, 4.0, SCALE, cb=8, nchunk=6, tau=1.0, phi=1.0, patience=0)
    np.testing.assert_array_equal(got["visited"], ref["keep"])
    np.testing.assert_allclose(got["out"], ref["out"], rtol=0, atol=1e-13)


def test_constant_values_stop_after_the_second_block():
    """Constant V: every probe equals v0's first channels, so both changes are 0
    and with patience 1 each stream stops right after its second kept block."""
    L, G = 4096, 4
    q, K, V = _case(L, G, seed=52)
    v0 = np.random.default_rng(3).standard_normal(128).astype(np.float16)
    Vc = np.broadcast_to(v0, (L, 128)).copy()
    pk = orc.quantize_k(K)
    r = orc.art_decode_head(q, pk, Vc, L, math.inf, SCALE, cb=8, nchunk=8, tau=1e-12, phi=1e-12, patience=1)
    for st in r["streams"]:
        assert st["visited"] == st["kept"][:2]
        assert all(ds < 1e-14 and dd < 1e-14 for ds, dd in st["steps"])
    np.testing.assert_allclose(r["out"], np.broadcast_to(v0.astype(np.float64), r["out"].shape), atol=1e-13)


def test_uniform_weights_follow_running_block_means():
    """q = 0 makes every score 0, so every block is kept and each chunk's
    running output is the plain mean of the values it has visited.  With
    blockwise-constant values u_b the probes are running means of u_b, whose
    changes shrink geometrically; the stop step follows in closed form."""
    L, G, cb, nchunk = 64 * 24, 2, 8, 3
    rng = np.random.default_rng(7)
    base = rng.standard_normal(128)
    rows = []
    for b in range(24):
        rows.append(np.broadcast_to(base + 0.5 ** (b // nchunk) * rng.standard_normal(128), (64, 128)))
    V = np.concatenate(rows).astype(np.float16)
    K = rng.standard_normal((L, 128)).astype(np.float16)
    q = np.zeros((G, 128), np.float16)
    pk = orc.quantize_k(K)
    tau, phi, p = 0.02, 2e-3, 2
    r = orc.art_decode_head(q, pk, V, L, 5.0, SCALE, cb=cb, nchunk=nchunk, tau=tau, phi=phi, patience=p)
    assert r["keep"].all()
    Vf = V.astype(np.float64)
    for c, st in enumerate(r["streams"]):
        blocks = [c + j * nchunk for j in range(cb)]
        means = np.cumsum(np.stack([Vf[64 * b, :8] for b in blocks]), axis=0) / np.arange(1, cb + 1)[:, None]
        stable, expect = 0, cb
        for t in range(1, cb):
            n1, n0 = np.linalg.norm(means[t]), np.linalg.norm(means[t - 1])
            stable = stable + 1 if (abs(n1 - n0) < tau and 1 - means[t] @ means[t - 1] / (n1 * n0) < phi) else 0
            if stable >= p:
                expect = t + 1
                break
        assert st["visited"] == blocks[:expect], f"chunk {c}"
    assert any(len(st["visited"]) < cb for st in r["streams"]), "case meant to stop some streams early"


def test_stop_is_monotone_in_patience_and_thresholds():
    L, G = 8192, 4
    q, K, V = _case(L, G, seed=53, needles=4)
    pk = orc.quantize_k(K)
    kw = dict(cb=16, nchunk=8)
    visits = {}
    for p in (1, 2, 4):
        for tau in (0.01, 0.05, 0.2):
            for phi in (1e-3, 1e-2):
                visits[(p, tau, phi)] = orc.art_decode_head(q, pk, V, L, math.inf, SCALE, tau=tau, phi=phi,
                                                            patience=p, **kw)["visited"]
    for (p, tau, phi), v in visits.items():
        for (p2, tau2, phi2), v2 in visits.items():
            if p2 >= p and tau2 <= tau and phi2 <= phi:
                assert (v <= v2).all(), ((p, tau, phi), (p2, tau2, phi2))
    assert visits[(1, 0.2, 1e-2)].sum() < visits[(4, 0.01, 1e-3)].sum(), "case too easy: nothing stops"


def test_visited_blocks_are_kept_and_streams_start_with_their_first_kept_block():
    L, G = 6000, 4
    q, K, V = _case(L, G, seed=54)
    pk = orc.quantize_k(K)
    r = orc.art_decode_head(q, pk, V, L, 3.0, SCALE, cb=4, nchunk=24, tau=0.1, phi=0.01, patience=1)
    assert (r["visited"] <= r["keep"]).all()
    union = sorted(b for st in r["streams"] for b in st["kept"])
    assert union == list(np.nonzero(r["keep"])[0])
    for st in r["streams"]:
        if st["kept"]:
            assert st["visited"][0] == st["kept"][0]
            assert st["visited"] == st["kept"][:len(st["visited"])]
    tok = np.repeat(r["visited"], 64)[:L]
    np.testing.assert_allclose(r["out"], orc.attend_tokens(r["s_exact"], V, np.nonzero(tok)[0]), atol=0)
