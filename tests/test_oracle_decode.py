"""Pins of the oracle's decode step (pseudo-max, Top-delta block selection, attention).

Checked against an exact-arithmetic brute force on tiny inputs, against
textbook softmax attention (scipy), and against invariants that follow from
"Faster Than Flash" (gist.science summary of arXiv 2609.00097), Method
section 2 (criterion s >= m~ - delta, pseudo-max over sink and local tokens)
and from the permutation invariance of online softmax.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import bruteforce as bf
from oracle import ffd_oracle as orc

SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def _case(L, G, seed, plant=True, vscale=1.0, needles=6):
    """Random keys with outlier channels; tokens 0..G-1 (one per head) and a few needles turned towards q."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, 128))
    K[:, rng.choice(128, 4, replace=False)] *= 5
    q = rng.standard_normal((G, 128)).astype(np.float16)
    if plant and L > 8:
        ns = min(G, L)
        pos = np.concatenate([np.arange(ns), rng.choice(np.arange(ns, L), min(needles, L - ns), replace=False)])
        for i, t in enumerate(pos):
            u = q[i % G].astype(np.float64)
            u /= np.linalg.norm(u)
            K[t] = np.linalg.norm(K[t]) * (0.9 * u + 0.1 * K[t] / np.linalg.norm(K[t]))
    V = (rng.standard_normal((L, 128)) * vscale).astype(np.float16)
    return q, K.astype(np.float16), V


@pytest.mark.parametrize("L,G,sink,local,delta", [
    (1, 1, 64, 256, 5.0), (63, 2, 64, 256, 5.0), (64, 4, 64, 256, 5.0), (65, 4, 8, 16, 2.0),
    (130, 7, 8, 16, 1.0), (321, 4, 64, 256, 5.0), (400, 2, 16, 32, 0.5), (400, 7, 64, 256, 3.0),
    (400, 4, 8, 16, 1.0),
])
def test_decode_head_matches_bruteforce(L, G, sink, local, delta):
    q, K, V = _case(L, G, seed=L * 10 + G, needles=2 if L == 400 else 6)
    ref = bf.decode_head([list(map(float, r)) for r in q], [list(map(float, r)) for r in K],
                         V.astype(np.float64).tolist(), L, delta, SCALE, sink, local)
    pk = orc.quantize_k(K)
    got = orc.decode_head(q, pk, V, L, delta, SCALE, sink, local)
    np.testing.assert_allclose(got["s_est"], np.array(ref["est"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["s_exact"], np.array(ref["exact"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["m_tilde"], ref["m_tilde"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["bmax"], np.array(ref["bmax"]).T, rtol=0, atol=1e-12)
    assert list(got["forced"]) == ref["forced"]
    assert list(got["keep"]) == ref["keep"]
    np.testing.assert_allclose(got["out"], np.array(ref["out"]), rtol=0, atol=1e-12)
    if (L, sink, local) in ((400, 16, 32), (400, 8, 16)):
        assert not all(ref["keep"]), "case meant to drop blocks keeps everything"


@pytest.mark.parametrize("L", [300, 1000, 4096])
def test_infinite_delta_is_dense_softmax_over_khat(L):
    q, K, V = _case(L, 4, seed=L)
    pk = orc.quantize_k(K)
    got = orc.decode_head(q, pk, V, L, np.inf, SCALE)
    assert got["keep"].all()
    _, khat = orc.dequantize(pk)
    s = (q.astype(np.float64) @ khat.T) * SCALE
    ref = softmax(s, axis=1) @ V.astype(np.float64)
    np.testing.assert_allclose(got["out"], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [1, 5, 64, 200, 320])
def test_short_sequences_are_dense_for_any_delta(L):
    """With L <= sink + local every block holds a support token, so all are forced."""
    q, K, V = _case(L, 2, seed=3 + L)
    pk = orc.quantize_k(K)
    dense = orc.decode_head(q, pk, V, L, np.inf, SCALE)["out"]
    for delta in (-1e30, 0.0, 1.0, 5.0):
        got = orc.decode_head(q, pk, V, L, delta, SCALE)
        assert got["keep"].all()
        np.testing.assert_array_equal(got["out"], dense)


def test_selection_monotone_in_delta_and_extremes():
    q, K, V = _case(4096, 4, seed=11)
    pk = orc.quantize_k(K)
    prev = None
    for delta in (-1e30, -3.0, 0.0, 1.0, 3.0, 5.0, 7.0, 10.0, np.inf):
        keep = orc.decode_head(q, pk, V, 4096, delta, SCALE)["keep"]
        if prev is not None:
            assert (keep >= prev).all(), delta          # keep(d1) subset of keep(d2) for d1 <= d2
        prev = keep
    lo = orc.decode_head(q, pk, V, 4096, -1e30, SCALE)
    np.testing.assert_array_equal(lo["keep"], lo["forced"])
    assert orc.decode_head(q, pk, V, 4096, np.inf, SCALE)["keep"].all()


def test_forced_blocks_always_kept_and_layout():
    for L in (1, 63, 64, 65, 319, 320, 321, 1000, 4096, 4097):
        f = orc.forced_blocks(L, 64, 256)
        nb = (L + 63) // 64
        assert f.shape == (nb,) and f[0] and f[-1]
        lo_blk = max(0, L - 256) // 64
        expect = np.zeros(nb, bool)
        expect[0] = True
        expect[lo_blk:] = True
        np.testing.assert_array_equal(f, expect)


def test_gqa_union_is_or_of_per_head_selections():
    q, K, V = _case(4096, 4, seed=21)
    pk = orc.quantize_k(K)
    full = orc.decode_head(q, pk, V, 4096, 3.0, SCALE)
    per = [orc.decode_head(q[h:h + 1], pk, V, 4096, 3.0, SCALE)["keep"] for h in range(4)]
    np.testing.assert_array_equal(full["keep"], np.logical_or.reduce(per))
    # thresholds are per query head
    np.testing.assert_allclose(full["thr"], full["m_tilde"] - 3.0)


def test_constant_values_and_single_token():
    q, K, V = _case(2000, 4, seed=5)
    pk = orc.quantize_k(K)
    v0 = np.random.default_rng(1).standard_normal(128).astype(np.float16)
    Vc = np.broadcast_to(v0, (2000, 128)).copy()
    out = orc.decode_head(q, pk, Vc, 2000, 5.0, SCALE)["out"]
    np.testing.assert_allclose(out, np.broadcast_to(v0.astype(np.float64), out.shape), rtol=0, atol=1e-13)
    one = orc.decode_head(q, pk, V, 1, 5.0, SCALE)["out"]
    np.testing.assert_array_equal(one, np.broadcast_to(V[0].astype(np.float64), one.shape))


@pytest.mark.parametrize("nsplit", [1, 3, 16])
def test_split_and_order_invariance_of_lse_merge(nsplit):
    q, K, V = _case(3000, 4, seed=9)
    pk = orc.quantize_k(K)
    r = orc.decode_head(q, pk, V, 3000, 4.0, SCALE)
    tok = np.nonzero(np.repeat(r["keep"], 64)[:3000])[0]
    rng = np.random.default_rng(nsplit)
    perm = rng.permutation(tok)
    parts = [orc.partial(r["s_exact"], V, p) for p in np.array_split(perm, nsplit)]
    parts.append(orc.partial(r["s_exact"], V, np.zeros(0, np.int64)))   # empty split is harmless
    np.testing.assert_allclose(orc.lse_merge(parts[::-1]), r["out"], rtol=0, atol=1e-12)


def test_dense_head_is_textbook_softmax():
    q, K, V = _case(777, 7, seed=2)
    got = orc.dense_head(q, K, V, 700, SCALE)
    s = (q.astype(np.float64) @ K[:700].astype(np.float64).T) * SCALE
    np.testing.assert_allclose(got, softmax(s, axis=1) @ V[:700].astype(np.float64), rtol=0, atol=1e-12)


def test_batch_wrapper_gqa_mapping():
    """Query head h reads KV head h // G."""
    rng = np.random.default_rng(4)
    B, Hkv, G, L = 2, 3, 2, 256
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, L, 128)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, L, 128)).astype(np.float16)
    pk = orc.quantize_cache(k)
    res = orc.decode(q, pk, v, [L, 100], 5.0, SCALE)
    for b in range(B):
        for h in range(Hkv):
            Lb = [L, 100][b]
            one = orc.decode_head(q[b, h * G:(h + 1) * G], orc.quantize_k(k[b, h]), v[b, h], Lb, 5.0, SCALE)
            np.testing.assert_array_equal(res[(b, h)]["out"], one["out"])


# ---- selection variants: per-head block sets and per-token masking ----

@pytest.mark.parametrize("select", ["head_block", "head_token"])
@pytest.mark.parametrize("L,G,sink,local,delta", [
    (130, 4, 8, 16, 1.0), (400, 4, 8, 16, 1.0), (400, 2, 16, 32, 0.5), (321, 7, 64, 256, 3.0),
])
def test_selection_variants_match_bruteforce(select, L, G, sink, local, delta):
    q, K, V = _case(L, G, seed=L * 7 + G, needles=6)
    ref = bf.decode_head([list(map(float, r)) for r in q], [list(map(float, r)) for r in K],
                         V.astype(np.float64).tolist(), L, delta, SCALE, sink, local, select=select)
    got = orc.decode_head(q, orc.quantize_k(K), V, L, delta, SCALE, sink, local, select=select)
    for h in range(G):
        assert list(np.nonzero(got["tmask"][h])[0]) == ref["attended"][h], f"head {h} token set"
    np.testing.assert_allclose(got["out"], np.array(ref["out"]), rtol=0, atol=1e-12)


def test_selection_variants_nest_and_union_is_the_block_filter():
    """head_token <= head_block <= union per head; the OR of the heads' block
    sets is the kept set; support tokens are always attended."""
    L, G, delta = 4096, 4, 3.0
    q, K, V = _case(L, G, seed=33)
    pk = orc.quantize_k(K)
    r = {s: orc.decode_head(q, pk, V, L, delta, SCALE, select=s) for s in orc.SELECTIONS}
    tu, tb, tt = r["union"]["tmask"], r["head_block"]["tmask"], r["head_token"]["tmask"]
    assert (tt <= tb).all() and (tb <= tu).all()
    assert tt.sum() < tb.sum() < tu.sum(), "case too easy: the variants coincide"
    blocks_any = np.zeros((L + 63) // 64, bool)
    for h in range(G):
        blocks_any |= tb[h].reshape(-1, 64).any(axis=1)
    np.testing.assert_array_equal(blocks_any, r["union"]["keep"])
    sup = orc.support_mask(L, 64, 256)
    assert tt[:, sup].all()
    # within a kept block a head_token head attends exactly the tokens at or above its threshold
    s_est, thr = r["head_token"]["s_est"], r["head_token"]["thr"]
    np.testing.assert_array_equal(tt[:, ~sup], (s_est >= thr[:, None])[:, ~sup])


def test_selection_variants_reduce_to_union_and_dense():
    L = 2000
    q, K, V = _case(L, 4, seed=41)
    pk = orc.quantize_k(K)
    dense = orc.decode_head(q, pk, V, L, math.inf, SCALE)["out"]
    for s in orc.SELECTIONS:
        np.testing.assert_allclose(orc.decode_head(q, pk, V, L, math.inf, SCALE, select=s)["out"], dense,
                                   rtol=0, atol=1e-13)
    # one query head per KV head: the head's block set is the kept set
    for h in range(4):
        a = orc.decode_head(q[h:h + 1], pk, V, L, 4.0, SCALE, select="head_block")
        u = orc.decode_head(q[h:h + 1], pk, V, L, 4.0, SCALE)
        np.testing.assert_array_equal(a["tmask"], u["tmask"])
        np.testing.assert_array_equal(a["out"], u["out"])


def test_selection_variants_monotone_in_delta():
    L = 3000
    q, K, V = _case(L, 4, seed=43)
    pk = orc.quantize_k(K)
    for s in ("head_block", "head_token"):
        prev = None
        for d in (0.5, 2.0, 5.0, 9.0):
            t = orc.decode_head(q, pk, V, L, d, SCALE, select=s)["tmask"]
            if prev is not None:
                assert (prev <= t).all(), f"{s}: delta {d} drops tokens kept at a smaller delta"
            prev = t
