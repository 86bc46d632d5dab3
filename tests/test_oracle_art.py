"""Pins of the oracle's run-time termination of the refine stream (the ART
page, "Attention Run-time Termination", Method sections 2.1-2.4, applied to
each stream of kept blocks; streams are contiguous runs of stream_blocks
blocks fixed by the call)."""
import math

import numpy as np
import pytest

from oracle import ffd_oracle as orc
from tests.test_oracle_decode import SCALE, _case


def test_streams_partition_the_sequence():
    for nblk, sb in [(64, 4), (100, 16), (5, 8), (257, 3), (1, 1), (4096, 16)]:
        lists = orc.art_streams(nblk, sb)
        assert len(lists) == math.ceil(nblk / sb)
        assert [b for l in lists for b in l] == list(range(nblk))
        assert all(1 <= len(l) <= sb and l == list(range(l[0], l[0] + len(l))) for l in lists)
        assert all(len(l) == sb for l in lists[:-1])
    with pytest.raises(ValueError):
        orc.art_streams(10, 0)


def test_disabled_stop_is_plain_decode():
    L, G = 3000, 4
    q, K, V = _case(L, G, seed=51)
    pk = orc.quantize_k(K)
    ref = orc.decode_head(q, pk, V, L, 4.0, SCALE)
    got = orc.art_decode_head(q, pk, V, L, 4.0, SCALE, stream_blocks=8, tau=1.0, phi=1.0, patience=0)
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
    r = orc.art_decode_head(q, pk, Vc, L, math.inf, SCALE, stream_blocks=8, tau=1e-12, phi=1e-12, patience=1)
    for st in r["streams"]:
        assert st["visited"] == st["kept"][:2]
        assert all(ds < 1e-14 and dd < 1e-14 for ds, dd in st["steps"])
    np.testing.assert_allclose(r["out"], np.broadcast_to(v0.astype(np.float64), r["out"].shape), atol=1e-13)


def test_uniform_weights_follow_running_block_means():
    """q = 0 makes every score 0, so every block is kept and each stream's
    running output is the plain mean of the values it has visited.  With
    blockwise-constant values u_b the probes are running means of u_b, whose
    changes shrink geometrically along each stream; the stop step follows in
    closed form."""
    L, G, sb = 64 * 24, 2, 8
    rng = np.random.default_rng(7)
    base = rng.standard_normal(128)
    rows = []
    for b in range(24):
        rows.append(np.broadcast_to(base + 0.5 ** (b % sb) * rng.standard_normal(128), (64, 128)))
    V = np.concatenate(rows).astype(np.float16)
    K = rng.standard_normal((L, 128)).astype(np.float16)
    q = np.zeros((G, 128), np.float16)
    pk = orc.quantize_k(K)
    tau, phi, p = 0.02, 2e-3, 2
    r = orc.art_decode_head(q, pk, V, L, 5.0, SCALE, stream_blocks=sb, tau=tau, phi=phi, patience=p)
    assert r["keep"].all()
    assert len(r["streams"]) == 3
    Vf = V.astype(np.float64)
    for c, st in enumerate(r["streams"]):
        blocks = list(range(c * sb, (c + 1) * sb))
        means = np.cumsum(np.stack([Vf[64 * b, :8] for b in blocks]), axis=0) / np.arange(1, sb + 1)[:, None]
        stable, expect = 0, sb
        for t in range(1, sb):
            n1, n0 = np.linalg.norm(means[t]), np.linalg.norm(means[t - 1])
            stable = stable + 1 if (abs(n1 - n0) < tau and 1 - means[t] @ means[t - 1] / (n1 * n0) < phi) else 0
            if stable >= p:
                expect = t + 1
                break
        assert st["visited"] == blocks[:expect], f"stream {c}"
    assert any(len(st["visited"]) < sb for st in r["streams"]), "case meant to stop some streams early"


def test_stop_is_monotone_in_patience_and_thresholds():
    L, G = 8192, 4
    q, K, V = _case(L, G, seed=53, needles=4)
    pk = orc.quantize_k(K)
    kw = dict(stream_blocks=16)
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
    r = orc.art_decode_head(q, pk, V, L, 3.0, SCALE, stream_blocks=4, tau=0.1, phi=0.01, patience=1)
    assert (r["visited"] <= r["keep"]).all()
    union = sorted(b for st in r["streams"] for b in st["kept"])
    assert union == list(np.nonzero(r["keep"])[0])
    for st in r["streams"]:
        if st["kept"]:
            assert st["visited"][0] == st["kept"][0]
            assert st["visited"] == st["kept"][:len(st["visited"])]
    tok = np.repeat(r["visited"], 64)[:L]
    np.testing.assert_allclose(r["out"], orc.attend_tokens(r["s_exact"], V, np.nonzero(tok)[0]), atol=0)


def test_streams_follow_the_call_not_the_batch_or_capacity():
    """The same sequence and query visit the same blocks and give the same
    output alone, inside a batch of 16 and at two cache capacities: the
    streams are fixed by the sequence and the call's stream_blocks."""
    L, G, sb = 2500, 4, 4
    q, K, V = _case(L, G, seed=55, needles=4)
    args = (3.0, SCALE, sb, 0.05, 0.01, 1)
    ref = orc.art_decode_head(q, orc.quantize_k(K), V, L, *args)
    rng = np.random.default_rng(56)
    for B, L_cap, b0 in [(1, 2560, 0), (16, 4096, 11), (16, 8192, 3)]:
        kq = (rng.standard_normal((B, 1, L_cap, 128))).astype(np.float16)
        vq = (rng.standard_normal((B, 1, L_cap, 128))).astype(np.float16)
        qq = (rng.standard_normal((B, G, 128))).astype(np.float16)
        kq[b0, 0, :L], vq[b0, 0, :L], qq[b0] = K[:L], V[:L], q
        lens = rng.integers(1, L_cap, size=B, endpoint=True)
        lens[b0] = L
        r = orc.art_decode(qq, orc.quantize_k(kq), vq, lens, *args, heads=[(b0, 0)])[(b0, 0)]
        np.testing.assert_array_equal(r["visited"], ref["visited"])
        np.testing.assert_array_equal(r["out"], ref["out"])
        assert [st["visited"] for st in r["streams"]] == [st["visited"] for st in ref["streams"]]
