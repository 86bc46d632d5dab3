"""GPU parity of the run-time termination of the refine streams
(ffd_decode_attn_ex with art_patience > 0) against the fp64 oracle.  Stream s
of a sequence is the contiguous run of art_stream_blocks blocks starting at
block s * art_stream_blocks; the oracle takes that length from the call.

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
ART_STREAM_BLOCKS_DEFAULT = 16


def _visited(got, b, h, G, L, label):
    """Blocks the GPU refined for (b, kv head h): token flags of the group's
    query heads, which must all agree."""
    nb = (L + 63) // 64
    tm = got["tmask"][b, h * G:(h + 1) * G, :L]
    assert (tm == tm[0]).all(), f"{label} query heads of a group visited different blocks"
    return tm[0, np.arange(nb) * 64] == 1


def _run_art(w, seed, delta, art, heads=None, stream_blocks=0):
    torch = torch_mod()
    tau, phi, patience = art
    sb = stream_blocks or ART_STREAM_BLOCKS_DEFAULT
    c = make_case(w, seed, heads=heads)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    say(f"art {w.name} seed={seed} delta={delta} stream_blocks={sb} art={art} heads={heads}")
    got = gpu_decode(shape, dev(c["q"], torch), cache, dev(c["seq_lens"], torch), delta, torch,
                     art=(tau, phi, patience, stream_blocks))
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
        visited = _visited(got, b, h, G, L, label)
        assert (visited <= keep).all(), f"{label} refined a dropped block"
        r = orc.art_decode_head(q16, pk, V16, L, delta, SM_SCALE, sb, tau, phi, patience, keep=keep)
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
    """delta = inf keeps every block; 16-block streams are long."""
    t = _run_art(WORKLOADS["tiny_h4x1_4k"], 0, math.inf, art, stream_blocks=16)
    if art[2] == 1:
        assert t["stopped"] > 0 and t["visited"] < t["kept"]


@pytest.mark.parametrize("seed", [1, 2])
def test_art_tiny_top_delta(seed):
    _run_art(WORKLOADS["tiny_h4x1_4k"], seed, 2.0, (0.05, 0.01, 1), stream_blocks=8)


@pytest.mark.parametrize("stream_blocks", [0, 4, 32])
def test_art_llama8b_16k(stream_blocks):
    """The 16K shape at the default stream length and at 4 and 32 blocks."""
    _run_art(WORKLOADS["llama8b_16k"], 0, 5.0, (0.05, 0.01, 1), heads=[(0, 0), (0, 5)],
             stream_blocks=stream_blocks)


def test_art_long_256k_sampled():
    t = _run_art(WORKLOADS["long_256k"], 0, 5.0, (0.05, 0.01, 1), heads=[(0, 2)])
    assert t["visited"] <= t["kept"]


def test_art_group_sizes_and_ragged_batch():
    _run_art(WORKLOADS["qwen7b_b16_16k32k"], 0, math.inf, (0.02, 0.005, 2), heads=[(4, 1)])
    for G, L, sb in [(1, 3000, 16), (8, 2500, 16), (3, 1000, 1), (5, 4000, 7)]:
        w = Workload(f"art_g{G}_l{L}", 2, 2 * G, 2, 4096, L, needles=4)
        _run_art(w, 0, math.inf, (0.05, 0.01, 1), stream_blocks=sb)


def test_art_streams_follow_the_call_not_the_batch_or_capacity():
    """The same sequences and queries visit the same blocks and give the same
    output bits alone (batch 1), inside a batch of 16, and at three cache
    capacities: the streams come from the call's stream length, not from the
    occupancy split of the launch.  The capacities have 12 to 256 streams per
    sequence, so the log-sum-exp merge runs in the one-wave kernel for up to
    64 partials and in the general one: both must give the same bits."""
    import sparse_long_context_ffd_amd as ffd
    torch = torch_mod()
    G, Hkv, L, delta, art = 4, 2, 3000, 3.0, (0.05, 0.01, 1, 4)
    w1 = Workload("art_same_b1", 1, G * Hkv, Hkv, 3008, L, needles=4)
    c1 = make_case(w1, 7)
    runs = []
    for B, L_cap, b0 in [(1, 3008, 0), (1, 8192, 0), (16, 4096, 9), (16, 8192, 2), (1, 32768, 0), (1, 65536, 0)]:
        rng = np.random.default_rng([B, L_cap])
        q = rng.standard_normal((B, G * Hkv, 128)).astype(np.float16)
        k = rng.standard_normal((B, Hkv, L_cap, 128)).astype(np.float16)
        v = rng.standard_normal((B, Hkv, L_cap, 128)).astype(np.float16)
        lens = rng.integers(1, L_cap, size=B, endpoint=True).astype(np.int32)
        q[b0], k[b0, :, :L], v[b0, :, :L], lens[b0] = c1["q"][0], c1["k"][0, :, :L], c1["v"][0, :, :L], L
        shape = ffd.make_shape(B, G * Hkv, Hkv, L_cap)
        cache = gpu_pack(shape, dev(k, torch), dev(v, torch))
        say(f"art same sequence: B={B} L_cap={L_cap} at b={b0} (plan {ffd.plan(shape)})")
        got = gpu_decode(shape, dev(q, torch), cache, dev(lens, torch), delta, torch, art=art)
        runs.append((got["out"][b0], [_visited(got, b0, h, G, L, f"B{B} L_cap{L_cap} h{h}") for h in range(Hkv)],
                     got["keep"][b0, :, :(L + 63) // 64].astype(bool)))
    out0, vis0, keep0 = runs[0]
    for out, vis, keep in runs[1:]:
        assert np.array_equal(keep, keep0), "kept blocks depend on the batch or the capacity"
        assert np.array_equal(out, out0), "output bits depend on the batch or the capacity"
        for a, b in zip(vis, vis0):
            assert np.array_equal(a, b), "visited blocks depend on the batch or the capacity"
    # and they are the oracle's
    for h in range(Hkv):
        pk = orc.quantize_k(c1["k"][0, h])
        r = orc.art_decode_head(c1["q"][0, h * G:(h + 1) * G], pk, c1["v"][0, h], L, delta, SM_SCALE, 4, *art[:3],
                                keep=keep0[h])
        robust = all(abs(ds - art[0]) > ART_BAND and abs(dd - art[1]) > ART_BAND
                     for st in r["streams"] for ds, dd in st["steps"])
        if robust:
            assert np.array_equal(vis0[h], r["visited"]), f"h{h}: visited blocks differ from the oracle's"
        d = out0[h * G:(h + 1) * G] - orc.decode_head(c1["q"][0, h * G:(h + 1) * G], pk, c1["v"][0, h], L, delta,
                                                      SM_SCALE, keep=vis0[h])["out"]
        assert np.abs(d).max() <= ATOL


def test_merge_of_more_than_64_live_partials():
    """A sequence with 79 live termination streams (more partials than the
    one-wave merge takes, so the general merge kernel runs) gives the same
    bits at capacities of 79 and 256 streams, and the oracle's output under
    the visited blocks."""
    import sparse_long_context_ffd_amd as ffd
    torch = torch_mod()
    G, Hkv, L, delta, art = 4, 2, 20000, 2.0, (0.05, 0.01, 1, 4)
    w1 = Workload("art_many_partials", 1, G * Hkv, Hkv, 20032, L, needles=8)
    c1 = make_case(w1, 11)
    outs = []
    for L_cap in (20032, 65536):
        k = np.zeros((1, Hkv, L_cap, 128), np.float16)
        v = np.zeros_like(k)
        k[:, :, :20032], v[:, :, :20032] = c1["k"], c1["v"]
        shape = ffd.make_shape(1, G * Hkv, Hkv, L_cap)
        cache = gpu_pack(shape, dev(k, torch), dev(v, torch))
        say(f"art many partials: L_cap={L_cap} (plan {ffd.plan(shape)})")
        got = gpu_decode(shape, dev(c1["q"], torch), cache, dev(c1["seq_lens"], torch), delta, torch, art=art)
        outs.append(got)
    assert np.array_equal(outs[0]["out"], outs[1]["out"]), "the output bits depend on the capacity"
    for h in range(Hkv):
        vis = _visited(outs[0], 0, h, G, L, f"h{h}")
        pk = orc.quantize_k(c1["k"][0, h])
        d = outs[0]["out"][0, h * G:(h + 1) * G] - orc.decode_head(c1["q"][0, h * G:(h + 1) * G], pk, c1["v"][0, h],
                                                                   L, delta, SM_SCALE, keep=vis)["out"]
        assert np.abs(d).max() <= ATOL
