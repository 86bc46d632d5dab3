"""The seeded synthetic workload generator: determinism, shapes, planted keys."""
import numpy as np
import pytest

from synthetic import WORKLOADS, make_case, make_head, planted_positions, seq_lens_for


def test_workloads_shapes_and_lengths():
    for w in WORKLOADS.values():
        assert w.max_len % 64 == 0 and w.q_heads % w.kv_heads == 0
        lens = seq_lens_for(w, 0)
        assert lens.shape == (w.batch,) and lens.dtype == np.int32
        assert (lens >= 1).all() and (lens <= w.max_len).all()
    lens = seq_lens_for(WORKLOADS["qwen7b_b16_16k32k"], 0)
    assert (lens >= 16384).all() and (lens <= 32768).all() and len(set(lens.tolist())) > 1
    assert (lens % 64 != 0).any()          # partial last blocks occur


def test_deterministic_and_slice_independent():
    w = WORKLOADS["tiny_h4x1_4k"]
    a = make_case(w, 3)
    b = make_case(w, 3)
    for k in ("q", "k", "v", "seq_lens"):
        np.testing.assert_array_equal(a[k], b[k])
    c = make_case(w, 4)
    assert not np.array_equal(a["k"], c["k"])
    q16, K16, V16 = make_head(w, 3, 0, 0, 4096)
    np.testing.assert_array_equal(K16, a["k"][0, 0])
    assert q16.dtype == K16.dtype == V16.dtype == np.float16


def test_planted_keys_cosine_and_positions():
    w = WORKLOADS["tiny_h4x1_4k"]
    L = 4096
    q16, K16, _ = make_head(w, 0, 0, 0, L)
    rng = np.random.default_rng([0, 0, 0])
    # replay the draws preceding the needle positions
    rng.standard_normal((w.max_len, 128)); rng.choice(128, size=4, replace=False)
    rng.standard_normal((w.max_len, 128)); rng.standard_normal((w.group, 128))
    pos = planted_positions(w, L, rng)
    assert list(pos[:4]) == [0, 1, 2, 3] and len(pos) == 4 + w.needles
    needles = pos[4:]
    assert len(set(needles.tolist())) == w.needles
    assert (needles >= w.sink).all() and (needles < L - w.local).all()
    for i, t in enumerate(pos):
        qd = q16[i % w.group].astype(np.float64)
        k = K16[t].astype(np.float64)
        cos = qd @ k / np.linalg.norm(qd) / np.linalg.norm(k)
        assert abs(cos - 0.8) < 2e-3


def test_stress_workload_has_no_planting_and_small_q():
    w = WORKLOADS["stress_b4_128k"]
    assert not w.plant and w.q_scale == 0.1 and w.needles == 0
