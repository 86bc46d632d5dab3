"""GPU parity of the run-time termination of each chunk's refine stream
(ffd_decode_attn_ex with art_patience > 0) against the fp64 oracle.

A stream's stop step follows from its sequence of (norm change, 1 - cosine)
values; where every one of the oracle's values lies farther than ART_BAND
from its threshold, the GPU (which decides in fp32) must visit exactly the
oracle's blocks.  Streams with a value inside the band are exempt.  The
output is compared with the oracle's attention over the blocks the GPU
actually refined (debug token flags), by the usual tolerances."""
import math

import numpy as np
import pytest

from oracle import ffd_oracle as orc
from synthetic import WORKLOADS, Workload, make_case
from tests.gpu_helpers import (ATOL, BAND, RTOL_L2, SM_SCALE, dev, gpu_decode, gpu_pack, mask_pins, say, shape_for,
                               torch_mod)

pytestmark = pytest.mark.gpu
ART_BAND = 1e-4


def _run_art(w, seed, delta, art, heads=None, chunk_blocks=0):
    import sparse_long_context_ffd_amd as ffd
    torch = torch_mod()
    tau, phi, patience = art
    c = make_case(w, seed, heads=heads)
    shape = shape_for(w, chunk_blocks)
    cb, nchunk = ffd.plan(shape)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    say(f"art {w.name} seed={seed} delta={delta} cb={cb} art={art} heads={heads}")
    got = gpu_decode(shape, dev(c["q"], torch), cache, dev(c["seq_lens"], torch), delta, torch, art=art)
    G = w.group
    todo = heads if heads is not None else [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    totals = {"streams": 0, "pinned": 0, "stopped": 0, "visited": 0, "kept": 0}
    for b, h in todo:
        L = int(c["seq_lens"][b])
        nb = (L + 63) // 64
        pk = orc.quantize_k(c["k"][b, h])
        q16, V16 = c["q"][b, h * G:(h + 1) * G], c["v"][b, h]
        label = f"{w.name} b{b} h{h}"
        base = orc.decode_head(q16, pk, V16, L, delta, SM_SCALE)
        keep = got["keep"][b, h, :nb].astype(bool)
        pkp, pdp = mask_pins(base)
        assert not (pkp & ~keep).any() and not (pdp & keep).any(), f"{label} mask mismatch on pinned blocks"
        assert np.abs(got["m_tilde"][b, h * G:(h + 1) * G] - base["m_tilde"]).max() <= BAND
        # blocks the GPU refined: token flags of the group's query heads (all equal)
        tm = got["tmask"][b, h * G:(h + 1) * G, :L]
        assert (tm == tm[0]).all(), f"{label} query heads of a group visited different blocks"
        first = np.arange(nb) * 64
        visited = tm[0, first] == 1
        assert (visited <= keep).all(), f"{label} refined a dropped block"
        r = orc.art_decode_head(q16, pk, V16, L, delta, SM_SCALE, cb, nchunk, tau, phi, patience, keep=keep)
        for st in r["streams"]:
            totals["streams"] += 1
            totals["stopped"] += len(st["visited"]) < len(st["kept"])
            robust = all(abs(ds - tau) > ART_BAND and abs(dd - phi) > ART_BAND for ds, dd in st["steps"])
            if robust:
                totals["pinned"] += 1
                gv = [b2 for b2 in st["kept"] if visited[b2]]
                assert gv == st["visited"], f"{label} stream {st['blocks'][:3]}...: GPU {gv} oracle {st['visited']}"
        totals["visited"] += int(visited.sum())
        totals["kept"] += int(keep.sum())
        ref = orc.decode_head(q16, pk, V16, L, delta, SM_SCALE, keep=visited)["out"]
        d = got["out"][b, h * G:(h + 1) * G] - ref
        max_abs, rel = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))
        assert max_abs <= ATOL and rel <= RTOL_L2, f"{label} output max-abs {max_abs} rel-L2 {rel}"
    say("  ", totals)
    assert totals["pinned"] >= 0.9 * totals["streams"], "too many streams near a threshold"
    return totals


@pytest.mark.parametrize("art", [(0.05, 0.01, 1), (0.02, 0.005, 2), (0.2, 0.05, 3)])
def test_art_tiny_long_streams(art):
    """delta = inf keeps every block; 16 blocks per chunk make long streams."""
    t = _run_art(WORKLOADS["tiny_h4x1_4k"], 0, math.inf, art, chunk_blocks=16)
    if art[2] == 1:
        assert t["stopped"] > 0 and t["visited"] < t["kept"]


@pytest.mark.parametrize("seed", [1, 2])
def test_art_tiny_top_delta(seed):
    _run_art(WORKLOADS["tiny_h4x1_4k"], seed, 2.0, (0.05, 0.01, 1), chunk_blocks=8)


def test_art_llama8b_16k_production_split():
    """The 16K shape in its production split (4 blocks per chunk): the stop
    logic runs after every refined block."""
    _run_art(WORKLOADS["llama8b_16k"], 0, 5.0, (0.05, 0.01, 1), heads=[(0, 0), (0, 5)])


def test_art_long_256k_sampled():
    t = _run_art(WORKLOADS["long_256k"], 0, 5.0, (0.05, 0.01, 1), heads=[(0, 2)])
    assert t["visited"] <= t["kept"]


def test_art_group_sizes_and_ragged_batch():
    _run_art(WORKLOADS["qwen7b_b16_16k32k"], 0, math.inf, (0.02, 0.005, 2), heads=[(4, 1)])
    for G, L in [(1, 3000), (8, 2500), (3, 1000)]:
        w = Workload(f"art_g{G}_l{L}", 2, 2 * G, 2, 4096, L, needles=4)
        _run_art(w, 0, math.inf, (0.05, 0.01, 1), chunk_blocks=16)
