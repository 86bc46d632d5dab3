"""GPU parity on a seeded random sweep of small decode problems: batch, KV
heads, group size, capacity, per-sequence lengths (ragged), support sizes,
delta (including "forced blocks only" and "keep everything"), forced chunk
sizes and the three selections, each checked against the fp64 oracle by the
rules of gpu_helpers (mask equal on pinned blocks, outputs within max-abs 2e-3
and rel-L2 1e-3 under the GPU's decisions).  The cases are drawn once from a
fixed seed, so a failure names a reproducible configuration."""
import math
import random

import pytest

from synthetic import Workload
from tests.test_gpu_decode import _run

pytestmark = pytest.mark.gpu


def _cases(n=64, seed=20261202):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        G = rng.randint(1, 8)
        hkv = rng.randint(1, 3)
        batch = rng.randint(1, 3)
        cap = 64 * rng.randint(1, 80)
        lo = rng.randint(1, cap)
        sink, local = rng.choice([(64, 256), (0, 64), (16, 0), (100, 300), (1, 1), (200, 40)])
        delta = rng.choice([-1e30, 0.5, 3.0, 7.0, math.inf])
        cap_cb = 32 if G <= 4 else 24
        cb = rng.choice([0, 0, rng.randint(1, cap_cb)])
        select = rng.choice(["union", "union", "head_block", "head_token"])
        out.append((i, G, hkv, batch, cap, lo, sink, local, delta, cb, select))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_small_problem(case):
    i, G, hkv, batch, cap, lo, sink, local, delta, cb, select = case
    w = Workload(f"rand{i}_g{G}_h{hkv}_b{batch}_cap{cap}", batch, G * hkv, hkv, cap, None, len_range=(lo, cap),
                 deltas=(delta,), needles=3, sink=sink, local=local)
    _run(w, i, [delta], chunk_blocks=cb, sink=sink, local=local, select=select)
