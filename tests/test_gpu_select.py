"""GPU parity of the selection variants (ffd_decode_attn_select): per-head
block sets and per-token masking inside the kept blocks, against the fp64
oracle.  Block masks, per-head token decisions (debug tmask) and outputs
follow the parity rules in gpu_helpers."""
import math

import numpy as np
import pytest

from synthetic import WORKLOADS, Workload
from tests.gpu_helpers import say
from tests.test_gpu_decode import _run

pytestmark = pytest.mark.gpu
SELECTS = ["head_block", "head_token"]


@pytest.mark.parametrize("select", SELECTS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_tiny(select, seed):
    st = _run(WORKLOADS["tiny_h4x1_4k"], seed, [5.0, 2.0, math.inf], select=select)
    assert all(s["attended_frac"] == 1.0 for s in st if s["delta"] == math.inf)
    say(f"{select} seed {seed}: attended {[round(s['attended_frac'], 4) for s in st]}")


@pytest.mark.parametrize("select", SELECTS)
def test_select_llama8b_16k_sampled(select):
    """The headline 16K shape (the production call, without debug buffers, must give the same bits)."""
    st = _run(WORKLOADS["llama8b_16k"], 0, [5.0], heads=[(0, 0), (0, 3), (0, 7)], select=select)
    assert all(s["attended_frac"] < s["keep_frac"] for s in st), "variant attends as much as the union"


@pytest.mark.parametrize("select", SELECTS)
def test_select_qwen_g7_ragged_sampled(select):
    """G = 7 (two column tiles of heads), ragged lengths, batch 16."""
    _run(WORKLOADS["qwen7b_b16_16k32k"], 0, [3.0], heads=[(2, 1), (11, 3)], select=select)


@pytest.mark.parametrize("select", SELECTS)
@pytest.mark.parametrize("cb", [1, 3])
def test_select_chunking_and_group_sizes(select, cb):
    _run(WORKLOADS["tiny_h4x1_4k"], 1, [3.0], chunk_blocks=cb, select=select)
    for G, L in [(1, 700), (8, 1000), (5, 65)]:
        w = Workload(f"sel_g{G}_l{L}", 2, 2 * G, 2, 2048, L, deltas=(2.0,), needles=4)
        _run(w, 0, [2.0, 0.5], select=select)


@pytest.mark.parametrize("select", SELECTS)
def test_select_sink_local_edges(select):
    w = WORKLOADS["tiny_h4x1_4k"]
    _run(w, 2, [2.0], sink=0, local=64, select=select)
    _run(w, 2, [2.0], sink=130, local=0, select=select)
    _run(w, 2, [1.0], sink=3, local=5, select=select)


def test_union_token_flags_cover_kept_blocks():
    """Under the default selection every valid token of a kept block is attended
    (check_head pins every union token flag)."""
    st = _run(WORKLOADS["tiny_h4x1_4k"], 0, [5.0])
    assert all(s["attended_frac"] is not None for s in st)
