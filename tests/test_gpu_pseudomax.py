"""GPU pseudo-max with maxima anywhere in the support set (no planted sinks).

The planted workloads put each head's largest support score on tokens 0..3;
here keys are unplanted, so the maximum can sit in any row of any tile of
the support blocks, and the pseudo-max must still match the oracle's.
"""
import pytest

from synthetic import Workload
from tests.test_gpu_decode import _run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("G,L", [(4, 4096), (7, 1000), (2, 333)])
def test_pseudomax_unplanted(seed, G, L):
    w = Workload(f"unplanted_g{G}_l{L}", 1, 2 * G, 2, 4096, L, deltas=(4.0,), needles=0, plant=False)
    _run(w, seed, [4.0])
