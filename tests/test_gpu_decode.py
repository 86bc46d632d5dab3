"""GPU parity of one FFD decode step (ffd_decode_attn) against the fp64 oracle.

Mask: equal on every pinned block; output: within max-abs 2e-3 and rel-L2
1e-3 of the oracle evaluated under the GPU's mask (rules in gpu_helpers).
"""
import math

import numpy as np
import pytest

from oracle import ffd_oracle as orc
from synthetic import WORKLOADS, Workload, make_case
from tests.gpu_helpers import (SM_SCALE, cache_to_host, check_head, dev, gpu_decode, gpu_dense, gpu_pack, say,
                               shape_for, torch_mod, ws_bytes)

pytestmark = pytest.mark.gpu


def _run(w, seed, deltas, heads=None, chunk_blocks=0, sink=None, local=None, fill=0xFF, select="union"):
    torch = torch_mod()
    c = make_case(w, seed, heads=heads)
    shape = shape_for(w, chunk_blocks, sink, local)
    S = w.sink if sink is None else sink
    W = w.local if local is None else local
    qd, kd, vd = dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch)
    ld = dev(c["seq_lens"], torch)
    cache = gpu_pack(shape, kd, vd, fill=fill)
    G = w.group
    todo = heads if heads is not None else [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    stats = []
    for delta in deltas:
        say(f"decode {w.name} seed={seed} delta={delta} cb={chunk_blocks} sink={S} local={W} select={select} "
            f"heads={todo}")
        got = gpu_decode(shape, qd, cache, ld, delta, torch, select=select)
        for b, h in todo:
            L = int(c["seq_lens"][b])
            pk = orc.quantize_k(c["k"][b, h])
            st = check_head(orc, c["q"][b, h * G:(h + 1) * G], pk, c["v"][b, h], L, delta, got, b, h, G,
                            sink=S, local=W, label=f"{w.name} s{seed} d{delta} b{b} h{h}", select=select)
            st.update(delta=delta, b=b, h=h)
            stats.append(st)
    for s in stats:
        say("  ", {k: (round(v, 7) if isinstance(v, float) else v) for k, v in s.items()})
    return stats


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_tiny(seed):
    st = _run(WORKLOADS["tiny_h4x1_4k"], seed, [5.0, 7.0, math.inf, -1e30])
    assert all(s["keep_frac"] == 1.0 for s in st if s["delta"] == math.inf)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_llama8b_16k_all_heads(seed):
    st = _run(WORKLOADS["llama8b_16k"], seed, [5.0, 7.0])
    kf = np.mean([s["keep_frac"] for s in st if s["delta"] == 5.0])
    say(f"llama8b_16k seed {seed} keep fraction at delta=5: {kf:.3f}")
    assert 0.0 < kf < 1.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_qwen_batched_sampled(seed):
    _run(WORKLOADS["qwen7b_b16_16k32k"], seed, [7.0, 3.0], heads=[(0, 0), (5, 3), (15, 1), (9, 2)])


@pytest.mark.parametrize("cb", [1, 3, 7, 11, 16, 25, 32])
def test_decode_chunking_invariance(cb):
    """The work split changes only the summation order.  On 64 blocks these
    chunk sizes give 1, 2, 3, 4, 6 and 8 thumbnail batches of 4 blocks per
    work-group (each a different path through the scan's loop and its peeled
    tail), with partial last batches at cb = 3, 7, 11 and 25."""
    _run(WORKLOADS["tiny_h4x1_4k"], 1, [5.0], chunk_blocks=cb)


@pytest.mark.parametrize("G,L", [(1, 1), (2, 63), (3, 64), (5, 65), (6, 320), (7, 321), (8, 1000), (4, 4031)])
def test_decode_group_sizes_and_ragged_lengths(G, L):
    """Every supported GQA group size, partial last blocks, L <= sink+local, NaN-filled cache tails."""
    w = Workload(f"g{G}_l{L}", 2, 2 * G, 2, 4096, L, deltas=(3.0,), needles=4)
    _run(w, 0, [3.0, 0.5], fill=0xFF)


@pytest.mark.parametrize("G,cb", [(5, 24), (8, 24), (7, 13)])
def test_decode_large_groups_at_the_chunk_cap(G, cb):
    """G > 4 at the largest chunk (24 blocks: 48-62 KB of estimates in LDS per
    work-group) and at a size with a partial last batch; 47 blocks in two or
    four chunks, so the chunks hold 23-24 and 11-12 blocks."""
    w = Workload(f"g{G}_cb{cb}", 2, 2 * G, 2, 3072, 3000, deltas=(3.0,), needles=4)
    _run(w, 0, [3.0], chunk_blocks=cb, fill=0xFF)


def test_decode_sink_and_local_variants():
    w = WORKLOADS["tiny_h4x1_4k"]
    _run(w, 2, [2.0], sink=0, local=64)
    _run(w, 2, [2.0], sink=130, local=0)
    _run(w, 2, [2.0], sink=0, local=1)


def test_decode_variable_lengths_in_batch():
    w = Workload("varlen", 4, 8, 2, 2048, None, len_range=(1, 2048), deltas=(4.0,), needles=3)
    _run(w, 5, [4.0])


def test_dense_matches_oracle():
    torch = torch_mod()
    for w, heads in [(WORKLOADS["tiny_h4x1_4k"], None), (WORKLOADS["llama8b_16k"], [(0, 1), (0, 6)]),
                     (Workload("dense_g7", 3, 14, 2, 1024, None, len_range=(1, 1024)), None)]:
        say(f"dense {w.name}")
        c = make_case(w, 0, heads=heads)
        shape = shape_for(w)
        out = gpu_dense(shape, dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch),
                        dev(c["seq_lens"], torch), torch)
        todo = heads if heads is not None else [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
        G = w.group
        for b, h in todo:
            L = int(c["seq_lens"][b])
            ref = orc.dense_head(c["q"][b, h * G:(h + 1) * G], c["k"][b, h], c["v"][b, h], L, SM_SCALE)
            d = out[b, h * G:(h + 1) * G] - ref
            ma, rel = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))
            say(f"  dense b{b} h{h} L{L} max_abs={ma:.2e} rel={rel:.2e}")
            assert ma <= 2e-3 and rel <= 1e-3


def test_decode_and_dense_share_a_workspace_across_splits():
    """At 64K context the decode splits into 6-block chunks and the dense
    baseline into 4-block ones.  One workspace of ffd_workspace_bytes serves
    both in turn; each matches the oracle and the decode repeats bit for bit."""
    import sparse_long_context_ffd_amd as ffd
    torch = torch_mod()
    w = Workload("split_64k", 1, 32, 8, 65536, 65536, needles=16)
    heads = [(0, 2), (0, 5)]
    c = make_case(w, 0, heads=heads)
    shape = shape_for(w)
    assert ffd.plan(shape)[0] == 6
    qd, kd, vd, ld = dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch), dev(c["seq_lens"], torch)
    cache = gpu_pack(shape, kd, vd)
    ws = torch.zeros(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    say(f"shared workspace {w.name}: decode, dense, decode")
    first = gpu_decode(shape, qd, cache, ld, 5.0, torch, ws=ws)
    dense = gpu_dense(shape, qd, kd, vd, ld, torch, ws=ws)
    again = gpu_decode(shape, qd, cache, ld, 5.0, torch, ws=ws)
    for k, v in first.items():
        assert np.array_equal(v, again[k], equal_nan=True), k
    G = w.group
    for b, h in heads:
        L = int(c["seq_lens"][b])
        pk = orc.quantize_k(c["k"][b, h])
        check_head(orc, c["q"][b, h * G:(h + 1) * G], pk, c["v"][b, h], L, 5.0, again, b, h, G,
                   sink=w.sink, local=w.local, label=f"split_64k b{b} h{h}")
        ref = orc.dense_head(c["q"][b, h * G:(h + 1) * G], c["k"][b, h], c["v"][b, h], L, SM_SCALE)
        d = dense[b, h * G:(h + 1) * G] - ref
        ma, rel = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))
        say(f"  dense b{b} h{h} max_abs={ma:.2e} rel={rel:.2e}")
        assert ma <= 2e-3 and rel <= 1e-3


def test_infinite_delta_equals_dense_over_khat():
    """delta = +inf keeps every block; the result is dense attention over K-hat."""
    torch = torch_mod()
    w = WORKLOADS["tiny_h4x1_4k"]
    c = make_case(w, 0)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    got = gpu_decode(shape, dev(c["q"], torch), cache, dev(c["seq_lens"], torch), math.inf, torch)
    assert (got["keep"][0, 0, :64] == 1).all()
    _, khat = orc.dequantize(orc.quantize_k(c["k"][0, 0]))
    ref = orc.dense_head(c["q"][0], khat, c["v"][0, 0], 4096, SM_SCALE)
    assert np.abs(got["out"][0] - ref).max() <= 2e-3


def test_decode_long_256k_sampled_heads():
    """Full 256K shape; oracle on sampled heads (the production call is
    required to give the same bits, gpu_helpers.gpu_decode)."""
    st = _run(WORKLOADS["long_256k"], 0, [5.0], heads=[(0, 0), (0, 7)])
    say(f"long_256k keep fractions: {[round(s['keep_frac'], 4) for s in st]}")


def test_decode_stress_128k_sampled_heads():
    """Low-sparsity stress shape (q x 0.1, nothing planted): most blocks kept."""
    st = _run(WORKLOADS["stress_b4_128k"], 0, [7.0], heads=[(1, 3), (3, 6)])
    assert all(s["keep_frac"] > 0.5 for s in st)


def test_graph_replay_matches_eager():
    """The decode step captured in a HIP graph (pseudo-max, fused kernel, merge)
    replays bit-identically to the eager call, several times, with eager work
    and synchronisations between replays."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    w = WORKLOADS["tiny_h4x1_4k"]
    c = make_case(w, 1)
    shape = shape_for(w)
    q, lens = dev(c["q"], torch), dev(c["seq_lens"], torch)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    ws = torch.empty(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out_e = torch.empty((1, 4, 128), dtype=torch.float16, device="cuda")
    ffd.decode_attn(shape, q, cache, lens, 5.0, SM_SCALE, out_e, ws)
    torch.cuda.synchronize()
    ref = out_e.clone()
    out_g = torch.zeros_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffd.decode_attn(shape, q, cache, lens, 5.0, SM_SCALE, out_g, ws)
    for r in range(4):
        out_g.zero_()
        junk = torch.randn(1 << 16, device="cuda").sum()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager result"
        assert torch.isfinite(junk)


def test_workspace_reuse_across_calls():
    """Calls in a row on one workspace with different queries each match the
    oracle, and a repeated query gives the same bits: nothing a call leaves in
    the workspace leaks into the next one."""
    torch = torch_mod()
    w = WORKLOADS["tiny_h4x1_4k"]
    c = make_case(w, 2)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    import sparse_long_context_ffd_amd as ffd
    ws = torch.full((ffd.workspace_bytes(shape),), 0x7F, dtype=torch.uint8, device="cuda")
    lens = dev(c["seq_lens"], torch)
    q2 = (np.random.default_rng(9).standard_normal(c["q"].shape) * 1.5).astype(np.float16)
    pk = orc.quantize_k(c["k"][0, 0])
    outs = []
    for r, q in enumerate((c["q"], q2, c["q"], q2, q2)):
        say(f"workspace reuse call {r}")
        got = gpu_decode(shape, dev(q, torch), cache, lens, 5.0, torch, ws=ws)
        check_head(orc, q[0], pk, c["v"][0, 0], 4096, 5.0, got, 0, 0, w.group, label=f"reuse call {r}")
        outs.append(got["out"])
    assert np.array_equal(outs[0], outs[2])
    assert np.array_equal(outs[1], outs[3]) and np.array_equal(outs[1], outs[4])


def test_workspace_shared_by_two_shapes():
    """One workspace used in turn by two shapes whose pseudo-max words overlap
    in memory: the sync words are keyed to the word layout, so neither shape
    takes the other's words (it computes the pseudo-max itself) and every call
    matches the oracle."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    wa = Workload("share_a", 1, 4, 1, 2048, 2048, deltas=(4.0,), needles=3)
    wb = Workload("share_b", 2, 8, 2, 1024, 1024, deltas=(4.0,), needles=3)
    cases = []
    for w in (wa, wb):
        c = make_case(w, 4)
        shape = shape_for(w)
        cases.append((w, c, shape, gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))))
    nbytes = max(ffd.workspace_bytes(sh) for _, _, sh, _ in cases)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for r in range(4):
        w, c, shape, cache = cases[r % 2]
        say(f"shared workspace call {r} ({w.name})")
        got = gpu_decode(shape, dev(c["q"], torch), cache, dev(c["seq_lens"], torch), 4.0, torch, ws=ws)
        G = w.group
        for b in range(w.batch):
            for h in range(w.kv_heads):
                pk = orc.quantize_k(c["k"][b, h])
                check_head(orc, c["q"][b, h * G:(h + 1) * G], pk, c["v"][b, h], int(c["seq_lens"][b]), 4.0, got,
                           b, h, G, label=f"shared call {r} b{b} h{h}")


def test_decode_loop_append_and_decode_in_one_graph():
    """Decode loop: one captured graph appends the step's key and value at each
    sequence's position L (ffd_append_kv), advances the device lengths, and runs
    the decode step; replayed step after step with new tokens and queries.  At
    every step the appended cache bytes equal the oracle's quantization and the
    output matches the oracle over the grown sequences (ragged batch, appends
    crossing a 64-token block and 4-token quads)."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    from tests.layout import decode_cache
    w = Workload("loop_b2_h8x2_2k", 2, 8, 2, 2048, None, len_range=(1000, 1500), needles=4)
    c = make_case(w, 3)
    B, Hq, Hkv, G, L_cap = w.batch, w.q_heads, w.kv_heads, w.group, w.max_len
    L0 = np.array([1021, 1497], np.int32)
    K, V = c["k"].copy(), c["v"].copy()
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(K, torch), dev(V, torch))
    pos = dev(L0, torch)
    k_new = torch.zeros((B, Hkv, 128), dtype=torch.float16, device="cuda")
    v_new = torch.zeros_like(k_new)
    q = torch.zeros((B, Hq, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros((B, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.empty(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    nb = L_cap // 64
    dbg = {"m_tilde": torch.zeros((B, Hq), dtype=torch.float32, device="cuda"),
           "bmax": torch.zeros((B, Hq, nb), dtype=torch.float32, device="cuda"),
           "keep": torch.zeros((B, Hkv, nb), dtype=torch.uint8, device="cuda")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffd.append_kv(shape, k_new, v_new, pos, cache)
        pos.add_(1)
        ffd.decode_attn(shape, q, cache, pos, 5.0, SM_SCALE, out, ws, debug=dbg)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), L0), "capture must not execute the graph"
    rng = np.random.default_rng(17)
    for i in range(6):
        kn = rng.standard_normal((B, Hkv, 128)).astype(np.float16)
        vn = rng.standard_normal((B, Hkv, 128)).astype(np.float16)
        qn = rng.standard_normal((B, Hq, 128)).astype(np.float16)
        k_new.copy_(torch.from_numpy(kn))
        v_new.copy_(torch.from_numpy(vn))
        q.copy_(torch.from_numpy(qn))
        out.fill_(float("nan"))
        dbg["keep"].fill_(7)
        torch.cuda.synchronize()
        say(f"decode loop step {i}")
        g.replay()
        torch.cuda.synchronize()
        L = L0 + i + 1
        assert np.array_equal(pos.cpu().numpy(), L)
        for b in range(B):
            K[b, :, L[b] - 1] = kn[b]
            V[b, :, L[b] - 1] = vn[b]
        got = {"out": out.float().cpu().numpy(), **{k: v.cpu().numpy() for k, v in dbg.items()}}
        raw = decode_cache(**cache_to_host(cache), B=B, Hkv=Hkv, L_cap=L_cap)
        for b in range(B):
            for h in range(Hkv):
                t = L[b] - 1
                ref = orc.quantize_k(kn[b, h][None])
                for f in ("codes", "scale", "zero", "res", "rscale"):
                    a, r = raw[f][b, h, t], ref[f][0]
                    if a.dtype == np.float16:
                        a, r = a.view(np.uint16), r.view(np.uint16)
                    assert np.array_equal(a, r), f"step {i} b{b} h{h}: appended {f} differs"
                assert np.array_equal(raw["v"][b, h, t].view(np.uint16), vn[b, h].view(np.uint16))
                pk = orc.quantize_k(K[b, h])
                check_head(orc, qn[b, h * G:(h + 1) * G], pk, V[b, h], int(L[b]), 5.0, got, b, h, G,
                           label=f"loop step {i} b{b} h{h}")


def test_dense_workspace_reuse_and_ragged_rows():
    """Dense calls in a row on one workspace with lengths that change the
    number of chunks per row between calls each match the oracle (nothing a
    call leaves in the workspace leaks into the next)."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    w = Workload("dense_reuse", 3, 12, 3, 2048, None, len_range=(1, 2048))
    c = make_case(w, 4)
    shape = shape_for(w, chunk_blocks=2)
    ws = torch.full((ffd.workspace_bytes(shape),), 0x7F, dtype=torch.uint8, device="cuda")
    qd, kd, vd = dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch)
    G = w.group
    for r, lens in enumerate(([2048, 1, 700], [64, 2047, 129], [1000, 1000, 1000])):
        say(f"dense reuse call {r} lens {lens}")
        ld = dev(np.array(lens, np.int32), torch)
        out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
        ffd.dense_decode_attn(shape, qd, kd, vd, ld, SM_SCALE, out, ws)
        got = out.float().cpu().numpy()
        for b in range(w.batch):
            for h in range(w.kv_heads):
                ref = orc.dense_head(c["q"][b, h * G:(h + 1) * G], c["k"][b, h], c["v"][b, h], lens[b], SM_SCALE)
                d = got[b, h * G:(h + 1) * G] - ref
                assert np.abs(d).max() <= 2e-3 and np.linalg.norm(d) <= 1e-3 * np.linalg.norm(ref), \
                    f"call {r} b{b} h{h}"


@pytest.mark.parametrize("q_scale,delta", [(8.0, 5.0), (8.0, math.inf), (0.01, 5.0), (0.01, -1e30)])
def test_decode_extreme_score_ranges(q_scale, delta):
    """Queries scaled so that the logits span hundreds of units (one key takes
    nearly all the weight; the refine's running maximum jumps by far more than
    its rescale slack) or almost nothing (near-uniform weights over every
    attended token): mask and output still match the oracle."""
    w = Workload(f"qscale{q_scale}", 2, 8, 2, 4096, None, len_range=(1500, 4096), deltas=(delta,), needles=6,
                 q_scale=q_scale)
    _run(w, 3, [delta])


def test_concurrent_calls_on_two_streams():
    """Two decode steps with their own workspaces enqueued on two streams
    without a synchronisation between them give the same bits as the same
    calls made one after the other: a call keeps all its state in its own
    workspace and outputs."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    wa = Workload("streams_a", 2, 16, 4, 8192, None, len_range=(3000, 8192), deltas=(5.0,), needles=6)
    wb = Workload("streams_b", 1, 28, 4, 16384, 16384, deltas=(7.0,), needles=8)
    runs = []
    for w, seed in ((wa, 1), (wb, 2)):
        c = make_case(w, seed)
        shape = shape_for(w)
        cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
        ws = torch.zeros(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
        runs.append((w, shape, dev(c["q"], torch), cache, dev(c["seq_lens"], torch), ws, out))
    # sequential reference (two calls each, so the second uses published words)
    ref = []
    for w, shape, q, cache, lens, ws, out in runs:
        for _ in range(2):
            ffd.decode_attn(shape, q, cache, lens, w.deltas[0], SM_SCALE, out, ws)
        torch.cuda.synchronize()
        ref.append(out.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        for (w, shape, q, cache, lens, ws, out), s in zip(runs, streams):
            out.zero_()
        torch.cuda.synchronize()
        for (w, shape, q, cache, lens, ws, out), s in zip(runs, streams):
            with torch.cuda.stream(s):
                ffd.decode_attn(shape, q, cache, lens, w.deltas[0], SM_SCALE, out, ws)
                ffd.decode_attn(shape, q, cache, lens, w.deltas[0], SM_SCALE, out, ws)
        torch.cuda.synchronize()
        for (w, shape, q, cache, lens, ws, out), r in zip(runs, ref):
            say(f"two streams rep {rep}: {w.name}")
            assert torch.equal(out, r), f"{w.name}: concurrent result differs from the sequential one"


def test_graph_replay_matches_eager_on_a_long_grid():
    """A decode step of a grid several times larger than the resident
    work-groups (where later chunks find the pseudo-max already published and
    decide while they scan) captured in a HIP graph: every replay, with eager
    work and synchronisations between them, gives the eager call's bits."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    w = Workload("graph_long", 4, 32, 8, 16384, None, len_range=(9000, 16384), deltas=(5.0,), needles=12)
    c = make_case(w, 6)
    shape = shape_for(w)
    cb, nch = ffd.plan(shape)
    assert nch * w.batch * w.kv_heads > 1024
    q, lens = dev(c["q"], torch), dev(c["seq_lens"], torch)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    ws = torch.zeros(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out_e = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
    for _ in range(2):
        ffd.decode_attn(shape, q, cache, lens, 5.0, SM_SCALE, out_e, ws)
    torch.cuda.synchronize()
    ref = out_e.clone()
    out_g = torch.zeros_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffd.decode_attn(shape, q, cache, lens, 5.0, SM_SCALE, out_g, ws)
    for r in range(4):
        out_g.zero_()
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"long-grid graph replay {r}")
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager result"
        assert torch.isfinite(junk)
    # and the result is the oracle's on a sampled head
    got = gpu_decode(shape, q, cache, lens, 5.0, torch)
    assert np.array_equal(got["out"], ref.float().cpu().numpy())
    pk = orc.quantize_k(c["k"][2, 5])
    check_head(orc, c["q"][2, 5 * w.group:6 * w.group], pk, c["v"][2, 5], int(c["seq_lens"][2]), 5.0, got, 2, 5,
               w.group, label="graph long b2 h5")


@pytest.mark.parametrize("G,cap,lens", [(4, 4096, [1, 70, 4096]), (7, 2048, [5, 2048])])
def test_stale_workspace_never_reaches_the_merge(G, cap, lens):
    """Every chunk of a launch writes its (m, l) -- a chunk past its sequence's
    end, or one that keeps nothing, with l = 0 -- so the merges read all of the
    launch's partials without waiting for the sequence lengths.  Rows far
    shorter than the capacity leave most chunks past their end.  With the
    workspace filled beforehand (all of it: the pseudo-max then takes its
    fallback; then all but the sync words: the in-grid hand-over) with bytes
    that read as a live partial (0x3F: m = l = 0.75) or as NaN (0xFF), each
    output must equal, bit for bit, the same call's on a zero-filled
    workspace: the production union step, the two selection variants,
    run-time termination and the dense baseline."""
    torch = torch_mod()
    import sparse_long_context_ffd_amd as ffd
    B = len(lens)
    w = Workload(f"stale_g{G}", B, 2 * G, 2, cap, None, len_range=(1, cap), needles=3)
    c = make_case(w, 7)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    qd, kd, vd = dev(c["q"], torch), dev(c["k"], torch), dev(c["v"], torch)
    ld = dev(np.array(lens, np.int32), torch)

    def run(fill, sync_kept, select="union", art=None, dense=False):
        n = ffd.workspace_bytes(shape) if dense else ws_bytes(shape, select, art)
        ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, w.q_heads, 128), dtype=torch.float16, device="cuda")
        call = (lambda: ffd.dense_decode_attn(shape, qd, kd, vd, ld, SM_SCALE, out, ws)) if dense else \
            (lambda: ffd.decode_attn(shape, qd, cache, ld, 5.0, SM_SCALE, out, ws, select=select, art=art))
        call()  # (initialises the sync words)
        ws[256 if sync_kept else 0:].fill_(fill)
        call()
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    for label, kw in [("union", {}), ("head_block", {"select": "head_block"}),
                      ("head_token", {"select": "head_token"}), ("art", {"art": (0.05, 0.01, 1, 4)}),
                      ("dense", {"dense": True})]:
        for sync_kept in (False, True):
            say(f"stale workspace G={G} lens={lens} {label} sync words kept={sync_kept}")
            ref = run(0x00, sync_kept, **kw)
            for fill in (0x3F, 0xFF):
                got = run(fill, sync_kept, **kw)
                assert np.isfinite(got).all(), f"{label}: non-finite output from a workspace of {fill:#x} bytes"
                assert np.array_equal(got, ref), f"{label}: output depends on the workspace's {fill:#x} bytes"
