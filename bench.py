#!/usr/bin/env python3
"""Benchmark one FFD decode-attention step on one MI355X; prints one JSON line.

A step is the whole hot path for one layer: pseudo-max, fused Top-delta scan +
refine, log-sum-exp merge, over inputs already resident in HBM: two kernel
launches, the pseudo-max work-groups leading the scan + refine launch
(ffd_plan_pseudomax; three launches where the pseudo-max has its own).  Defaults: the Llama-3.1-8B-like 16K decode layer (B=1, Hq=32, Hkv=8,
delta=5), plus the 256K long-context shape with the in-house dense
flash-decode kernel timed beside it.

Timing: the decode step is captured in a HIP graph, as the pages do with
CUDA graphs to remove CPU launch overhead: W untimed warm-up steps, then one
graph of exactly K steps replayed between two events and bracketed by
torch.cuda.synchronize().  The 256 MB last-level cache (MALL) is defeated two
ways: per-layer caches are rotated (step i reads copy i mod R), with R sized
from the bytes one step reads so that more than 1.1 GB is read between two
visits of one copy (R = ceil(1.1 GB / bytes per step) + 1), and before every
timed replay a 1 GiB device copy (1 GiB read, 1 GiB written) evicts what the
previous replay left, outside the events.  The fused scan + refine kernel is then timed
alone: a graph of K back-to-back launches of it (stage mask 2) on the same
stream; its mean launch duration is the roofline denominator.  When the
pseudo-max runs inside that launch it needs the merge of the same step (which
advances the tag of the published maxima), so its duration is taken as the
mean of K (scan + refine, merge) launch pairs minus that of K merges alone.  Eager
(uncaptured) launches are timed too and reported as eager_us_per_step.  The
K-step graph is replayed REPLAYS - 1 more times for us_per_step_spread (p10,
median, p90 of the per-replay means; `value` is the first replay).

cache_warm_us_per_step: the same K steps on one layer's cache, without the
rotation, so part of it stays in the last-level cache (labelled, never `value`).

Achievable HBM (hbm_achievable): the library's streaming-read kernel over 1 GiB
and a 1 GiB device-to-device copy, timed with events, reported beside the
nominal peak.

Roofline: achieved = algorithmic bytes of the fused kernel per launch (48 B per
token-head scanned + 392 B per kept token-head refined, + 184 B per support
token-head when the pseudo-max runs inside it) / its mean duration, against
the 8 TB/s HBM3E peak.

Legs beside the headline 16K step (all timed the same way):
  long_context   the 256K shape (delta 5) and the dense baseline; its
                 scan_only object is the same shape at delta = -1e30 (only the
                 forced sink/local blocks refined), so the attend kernel is
                 almost only the 2-bit thumbnail stream;
  batched_qwen   the batch of 16 Qwen2.5-7B-like heads at 16K-32K (delta 7);
  stress         the low-sparsity B=4 x 128K shape (delta 7);
  context_sweep  FFD and dense at 16K, 32K, 64K, 128K and 256K with the
                 Llama-8B-like heads, with least-squares slopes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
SCAN_BYTES = 48      # 2-bit codes 32 B + (scale, zero) 16 B per token-head
REFINE_BYTES = 392   # int8 residual 128 B + rscale 8 B + fp16 V 256 B per kept token-head
PSEUDO_BYTES = 184   # packed K (codes, scale/zero, residual, rscale) per support token-head
DENSE_BYTES = 512    # fp16 K + V per token-head
TOUCH_BETWEEN_VISITS = 1.1e9  # bytes read between two visits of one rotated cache copy
ROTATE_BUDGET = 48e9          # device bytes the rotated copies of one leg may take
FLUSH_BYTES = 1 << 30         # the pre-replay copy: 1 GiB read + 1 GiB written
# HBM bytes per launch of the fused kernel, from two rocprofv3 --pmc passes over
# `bench.py --workload W --no-long --no-variants --no-cpu-baseline --steps 20 --warmup 5`
# (FETCH_SIZE, then WRITE_SIZE: KiB per dispatch, median over the dispatches of
# the attend kernel the step runs, the launch with diagnostic outputs left out).  Both counters are scaled by what they read for the plain
# 256 MiB device-to-device copy bench.py does first: FETCH_SIZE read 131088.6 KiB
# for 262144 KiB moved (x2.0), WRITE_SIZE 262144 KiB (x1.0).  An entry counts only
# while the kernel sources hash to the digest it was recorded with.
FETCH_SCALE, WRITE_SCALE = 262144 / 131088.6, 1.0
TRAFFIC_KIB = {
    "llama8b_16k": {"sources": "dfbc5751e1d193e9", "fetch": 10225.75, "write": 695.5},
    "long_256k": {"sources": "dfbc5751e1d193e9", "fetch": 133826.44, "write": 2465.94},
    "qwen7b_b16_16k32k": {"sources": "dfbc5751e1d193e9", "fetch": 338044.16, "write": 5288.2},
    "stress_b4_128k": {"sources": "dfbc5751e1d193e9", "fetch": 902841.72, "write": 4382.78},
}
REPLAYS = 10  # replays of the K-step graph behind the reported spread (the first is the timed one)
METRIC = "decode-attn µs/step + effective HBM GB/s vs peak, 16K–256K ctx"


def kernel_digest() -> str:
    """sha256 over the code (comments and whitespace removed) of the HIP
    sources, the public header and the build script: a change of comments
    leaves the kernels, and so the recorded counters, as they are."""
    import hashlib
    import re
    pkg = os.path.join(ROOT, "sparse_long_context_ffd_amd")
    files = sorted(os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc")))
    files += [os.path.join(pkg, "build.py"), os.path.join(ROOT, "include", "ffd.h")]
    h = hashlib.sha256()
    for f in files:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        if f.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
        else:
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(os.path.basename(f).encode())
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_bytes(workload: str):
    """Profiled HBM bytes per fused-kernel launch, or None when none were
    recorded for this workload with the current kernel sources."""
    t = TRAFFIC_KIB.get(workload)
    if t is None or t["sources"] != kernel_digest():
        return None
    return int(round((t["fetch"] * FETCH_SCALE + t["write"] * WRITE_SCALE) * 1024))


def graph_of(calls, torch):
    """Capture a list of zero-argument launch callables into one HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def copies_for(read_bytes_per_step: int, stored_bytes: int) -> int:
    """Rotated cache copies R: more than TOUCH_BETWEEN_VISITS bytes are read
    between two visits of one copy when R - 1 steps run in between, within
    ROTATE_BUDGET of device memory (never fewer than 2)."""
    r = math.ceil(TOUCH_BETWEEN_VISITS / max(int(read_bytes_per_step), 1)) + 1
    cap = max(2, int(ROTATE_BUDGET // max(int(stored_bytes), 1)))
    return int(max(2, min(r, cap, 512)))


class Flush:
    """Evicts the last-level cache between timed replays: a device-to-device
    copy of FLUSH_BYTES (its own 2 GiB of buffers, read and written once)."""

    def __init__(self, torch):
        self.src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.dst.copy_(self.src)


def timed_replay(g, torch, flush=None) -> float:
    """Replay a captured graph between two events (after `flush`, outside the
    events); returns milliseconds."""
    torch.cuda.synchronize()
    if flush is not None:
        flush()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def hbm_probe(torch, mib=1024, reps=5):
    """Achievable HBM rate on this device, beside the nominal peak: the best of
    `reps` timed runs of the library's streaming-read kernel (ffd_stream_read,
    read bytes) and of a plain device-to-device copy (read + write bytes), each
    over `mib` MiB (above the 256 MB MALL, so the source is not cache-resident)."""
    import sparse_long_context_ffd_amd as ffd
    n = mib << 20
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.empty(ffd._lib.STREAM_READ_SINK_BYTES, dtype=torch.uint8, device="cuda")

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    t_copy = best(lambda: dst.copy_(src))
    t_read = best(lambda: ffd.stream_read(src, sink))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbps": round(2 * n / (t_copy * 1e6), 1), "read_gbps": round(n / (t_read * 1e6), 1),
            "bytes": n, "peak_gbps": HBM_PEAK_GBPS,
            "how": f"best of {reps}: ffd_stream_read (read bytes) and a torch device-to-device copy "
                   f"(read + write bytes), {mib} MiB each"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prepare(w, seed, torch):
    from synthetic import make_case
    t0 = time.time()
    c = make_case(w, seed)
    log(f"generated {w.name} in {time.time() - t0:.1f}s")
    return c, {k: to_dev(v, torch) for k, v in c.items()}


def measure_ffd(w, delta, steps, warmup, c, d, torch, sm_scale, flush, with_variants=False, extras=True):
    """Time the FFD decode step of workload `w` (graph of `steps` steps over
    rotated cache copies) and its attend kernel alone; with `extras` also the
    eager launches, the decode loop with append, and the cache-warm step."""
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len, sink=w.sink, local=w.local)
    base = ffd.PackedCache(shape)
    ffd.quantize_k(shape, d["k"], 0, w.max_len, base)
    ffd.pack_v(shape, d["v"], 0, w.max_len, base)
    ws = torch.empty(max(ffd.workspace_bytes(shape), ffd.workspace_bytes_ex(shape, art=ART)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
    nb = w.max_len // 64
    keep = torch.zeros((w.batch, w.kv_heads, nb), dtype=torch.uint8, device="cuda")
    ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, out, ws, debug={"keep": keep})
    torch.cuda.synchronize()
    keep = keep.cpu().numpy().astype(bool)
    lens = c["seq_lens"].astype(np.int64)
    tok_total = int(lens.sum()) * w.kv_heads
    kept_tok = 0
    for b in range(w.batch):
        L = int(lens[b])
        nbb = (L + 63) // 64
        per_tok = np.repeat(keep[b, :, :nbb], 64, axis=1)[:, :L]
        kept_tok += int(per_tok.sum())
    keep_frac = kept_tok / tok_total
    attend_bytes = SCAN_BYTES * tok_total + REFINE_BYTES * kept_tok
    support = sum(min(int(L), w.sink + w.local) for L in lens) * w.kv_heads
    step_bytes = attend_bytes + PSEUDO_BYTES * support
    _, pm_in_grid = ffd.plan_pseudomax(shape)
    if pm_in_grid:  # the pseudo-max work-groups are part of the attend launch
        attend_bytes += PSEUDO_BYTES * support

    layer_bytes = sum(n for n in ffd.cache_bytes(shape).values())
    R = copies_for(step_bytes, layer_bytes)
    layers = [base] + [base.clone() for _ in range(R - 1)]
    log(f"ffd {w.name} delta={delta}: keep={keep_frac:.4f} reads {step_bytes / 1e6:.1f} MB/step, rotate R={R} "
        f"({R * layer_bytes / 1e9:.2f} GB stored, {(R - 1) * step_bytes / 1e9:.2f} GB read between visits)")

    def step(i, stages=0, select="union", art=None):
        ffd.decode_attn(shape, d["q"], layers[i % R], d["seq_lens"], delta, sm_scale, out, ws,
                        debug={"stages": stages} if stages else None, select=select, art=art)

    res = {}
    if extras:
        # eager launches (host-bound for short contexts), for reference
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        flush()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            step(i)
        t1.record()
        torch.cuda.synchronize()
        res["eager_us_per_step"] = t0.elapsed_time(t1) * 1e3 / steps
    # the decode step as the pages run it: captured in a graph (K steps over the
    # rotated layers per replay); W warm-up steps replayed first
    g_warm, g_steps = graph_of([lambda i=i: step(i) for i in range(warmup)], torch), \
        graph_of([lambda i=i: step(i) for i in range(steps)], torch)
    if pm_in_grid:
        g_attend = graph_of([lambda i=i: step(i, stages=6) for i in range(steps)], torch)
        g_merge = graph_of([lambda i=i: step(i, stages=4) for i in range(steps)], torch)
    else:
        g_attend = graph_of([lambda i=i: step(i, stages=2) for i in range(steps)], torch)
        g_merge = None
    g_warm.replay()
    g_steps.replay()  # untimed: a graph's first launch also uploads it to the device
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms = timed_replay(g_steps, torch, flush)
    wall = time.perf_counter() - wall0
    # spread: the same K-step graph replayed again, one mean per replay
    rep_us = sorted([total_ms * 1e3 / steps] + [timed_replay(g_steps, torch, flush) * 1e3 / steps
                                                 for _ in range(REPLAYS - 1)])
    g_attend.replay()
    attend_total_ms = timed_replay(g_attend, torch, flush)
    if g_merge is not None:
        g_merge.replay()
        attend_total_ms -= timed_replay(g_merge, torch, flush)
    del g_warm, g_attend, g_merge
    if extras:
        # decode loop: each step first appends one token per sequence (its last
        # one, rewritten with the same key and value, so the cache and the work
        # stay fixed)
        last = d["seq_lens"].long() - 1
        bidx = torch.arange(w.batch, device="cuda")
        k_last = d["k"][bidx, :, last].contiguous()          # [B][Hkv][128]
        v_last = d["v"][bidx, :, last].contiguous()
        pos = (d["seq_lens"] - 1).to(torch.int32).contiguous()

        def loop_step(i):
            ffd.append_kv(shape, k_last, v_last, pos, layers[i % R])
            step(i)

        g_loop = graph_of([lambda i=i: loop_step(i) for i in range(steps)], torch)
        g_loop.replay()
        res["loop_us_per_step"] = timed_replay(g_loop, torch, flush) * 1e3 / steps
        del g_loop
        # the same K steps on one layer's cache (no rotation, no flush): the
        # cache-warm time, with the layer's bytes partly resident in the MALL
        g_warmcache = graph_of([lambda: ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, out,
                                                        ws) for _ in range(steps)], torch)
        g_warmcache.replay()
        res["cache_warm_us_per_step"] = timed_replay(g_warmcache, torch) * 1e3 / steps
        del g_warmcache
    us_step = total_ms * 1e3 / steps
    attend_us = attend_total_ms * 1e3 / steps
    variants = selection_variants(shape, w, delta, d, base, ws, sm_scale, torch, steps, step, flush) \
        if with_variants else None
    res.update({
        "variants": variants,
        "us_per_step": us_step,
        "replay_spread": {"replays": REPLAYS, "p10": round(float(np.percentile(rep_us, 10)), 3),
                          "median": round(float(np.median(rep_us)), 3),
                          "p90": round(float(np.percentile(rep_us, 90)), 3)},
        "wall_us_per_step": wall * 1e6 / steps,
        "attend_us_mean": attend_us,
        "pm_in_grid": pm_in_grid,
        "keep_fraction": keep_frac,
        "attend_bytes": attend_bytes,
        "step_bytes": step_bytes,
        "tokens": tok_total,
        "layers_rotated": R,
        "read_between_visits": (R - 1) * step_bytes,
        "plan": ffd.plan(shape),
    })
    return res


# run-time termination timed beside the selection variants: (tau, phi,
# patience, stream length); streams of 4 blocks give the 16K step as many
# work-groups as the union split
ART = (0.05, 0.01, 1, 4)


def selection_variants(shape, w, delta, d, cache, ws, sm_scale, torch, steps, step, flush):
    """Per-head block sets, per-token masking and run-time termination: time
    per step, fraction of (query head, token) pairs attended, and the output's
    deviation from full attention over K-hat (delta = +inf).  The selection
    variants load the kept blocks' bytes; termination skips some of them."""
    import sparse_long_context_ffd_amd as ffd
    rows = (w.batch, w.q_heads, 128)
    full = torch.empty(rows, dtype=torch.float16, device="cuda")
    ffd.decode_attn(shape, d["q"], cache, d["seq_lens"], math.inf, sm_scale, full, ws)
    lens = d["seq_lens"].long()
    valid = torch.arange(w.max_len, device="cuda")[None, :] < lens[:, None]          # [B][L_cap]
    res = {}
    for sel in ("union", "head_block", "head_token", "art"):
        o = torch.empty(rows, dtype=torch.float16, device="cuda")
        tm = torch.zeros((w.batch, w.q_heads, w.max_len), dtype=torch.uint8, device="cuda")
        kw = {"art": ART} if sel == "art" else {"select": sel}
        ffd.decode_attn(shape, d["q"], cache, d["seq_lens"], delta, sm_scale, o, ws, debug={"tmask": tm}, **kw)
        torch.cuda.synchronize()
        att = ((tm == 1) & valid[:, None, :]).sum().item() / (valid.sum().item() * w.q_heads)
        diff = (o.float() - full.float())
        g = graph_of([lambda i=i: step(i, **kw) for i in range(steps)], torch)
        g.replay()
        us = timed_replay(g, torch, flush) * 1e3 / steps
        res[sel] = {**({"tau_phi_patience_stream_blocks": list(ART)} if sel == "art" else {}),
                    "us_per_step": round(us, 3), "attended_frac": round(att, 5),
                    "max_abs_vs_full": round(diff.abs().max().item(), 6),
                    "rel_l2_vs_full": round((diff.norm() / full.float().norm()).item(), 6)}
        del g
    return res


def measure_dense(w, steps, warmup, d, torch, sm_scale, flush):
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len, sink=w.sink, local=w.local)
    ws = torch.empty(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
    layer_bytes = (d["k"].numel() + d["v"].numel()) * 2
    byts = DENSE_BYTES * int(d["seq_lens"].sum().item()) * w.kv_heads
    R = copies_for(byts, layer_bytes)
    ks = [d["k"]] + [d["k"].clone() for _ in range(R - 1)]
    vs = [d["v"]] + [d["v"].clone() for _ in range(R - 1)]

    def step(i):
        ffd.dense_decode_attn(shape, d["q"], ks[i % R], vs[i % R], d["seq_lens"], sm_scale, out, ws)

    g_warm = graph_of([lambda i=i: step(i) for i in range(warmup)], torch)
    g_steps = graph_of([lambda i=i: step(i) for i in range(steps)], torch)
    g_warm.replay()
    g_steps.replay()  # untimed: a graph's first launch also uploads it to the device
    us = timed_replay(g_steps, torch, flush) * 1e3 / steps
    del ks, vs, g_warm, g_steps
    return {"us_per_step": us, "bytes": byts, "gbps": byts / us / 1e3, "layers_rotated": R,
            "read_between_visits": (R - 1) * byts}


def measure_split(w, delta, steps, warmup, c, d, torch, sm_scale, flush):
    """The split path of the same step (debug split_mode 2: a scan kernel that
    writes keep bitmaps, then a refine kernel over the compacted kept blocks):
    whole step, scan kernel alone and refine kernel alone, each a graph of
    `steps` launches over rotated copies, with their algorithmic bytes (48 B
    per token-head scanned; 440 B per kept token-head refined: residual 128 +
    rscale 8 + V 256 + the thumbnail read again, 48)."""
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len, sink=w.sink, local=w.local)
    base = ffd.PackedCache(shape)
    ffd.quantize_k(shape, d["k"], 0, w.max_len, base)
    ffd.pack_v(shape, d["v"], 0, w.max_len, base)
    ws = torch.empty(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float16, device="cuda")
    nb = w.max_len // 64
    keep = torch.zeros((w.batch, w.kv_heads, nb), dtype=torch.uint8, device="cuda")
    ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, out, ws,
                    debug={"keep": keep, "split_mode": 2, "pm_mode": 1})
    torch.cuda.synchronize()
    keep = keep.cpu().numpy().astype(bool)
    lens = c["seq_lens"].astype(np.int64)
    tok_total = int(lens.sum()) * w.kv_heads
    kept_tok = sum(int(np.repeat(keep[b, :, :(int(L) + 63) // 64], 64, axis=1)[:, :int(L)].sum())
                   for b, L in enumerate(lens))
    scan_bytes, refine_bytes = SCAN_BYTES * tok_total, (REFINE_BYTES + SCAN_BYTES) * kept_tok
    layer_bytes = sum(n for n in ffd.cache_bytes(shape).values())
    R = copies_for(scan_bytes + refine_bytes, layer_bytes)
    layers = [base] + [base.clone() for _ in range(R - 1)]

    def step(i, stages=0):
        ffd.decode_attn(shape, d["q"], layers[i % R], d["seq_lens"], delta, sm_scale, out, ws,
                        debug={"split_mode": 2, "pm_mode": 1, "stages": stages})

    step(0)
    res = {}
    for name, st in (("step", 0), ("scan", 8), ("refine", 16)):
        g = graph_of([lambda i=i: step(i, st) for i in range(steps)], torch)
        g.replay()
        res[name] = timed_replay(g, torch, flush) * 1e3 / steps
        del g
    del layers, base
    rf = lambda byts, us: {"achieved": round(byts / (us * 1e3), 1), "frac": round(byts / (us * 1e3) / HBM_PEAK_GBPS, 4),
                           "bytes_per_launch": byts, "kernel_us": round(us, 3)}
    return {"us_per_step": round(res["step"], 3), "scan_kernel": rf(scan_bytes, res["scan"]),
            "refine_kernel": rf(refine_bytes, res["refine"]), "layers_rotated": R,
            "note": "debug split_mode 2 (not the default path: slower than the fused kernel here)"}


def roofline_of(r, workload):
    """The attend kernel's roofline entry of one measure_ffd result."""
    ach = r["attend_bytes"] / (r["attend_us_mean"] * 1e3)
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic_bytes(workload),
            "bytes_per_launch": r["attend_bytes"], "attend_kernel_us": round(r["attend_us_mean"], 3)}


def leg(name, w, delta, steps, warmup, seed, torch, sm_scale, flush, dense=True, scan_only=False, split=False):
    """One workload beside the headline: FFD step and attend kernel (roofline),
    the dense baseline, and optionally the scan-only variant (delta = -1e30)."""
    c, d = prepare(w, seed, torch)
    r = measure_ffd(w, delta, steps, warmup, c, d, torch, sm_scale, flush, extras=False)
    out = {"workload": w.name, "delta": delta, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
           "seq_len_max": int(c["seq_lens"].max()), "tokens_per_kv_head": int(c["seq_lens"].sum()),
           "us_per_step": round(r["us_per_step"], 3), "us_per_step_spread": r["replay_spread"],
           "keep_fraction": round(r["keep_fraction"], 5),
           "effective_gbps": round(r["step_bytes"] / (r["us_per_step"] * 1e3), 1),
           "kv_tokens_per_s": r["tokens"] / (r["us_per_step"] * 1e-6),
           "context_tokens_per_s": r["tokens"] / w.kv_heads / (r["us_per_step"] * 1e-6),
           "roofline_attend": roofline_of(r, w.name), "layers_rotated": r["layers_rotated"],
           "read_between_visits_gb": round(r["read_between_visits"] / 1e9, 3), "chunk_blocks": r["plan"][0]}
    if scan_only:
        so = measure_ffd(w, -1e30, steps, warmup, c, d, torch, sm_scale, flush, extras=False)
        out["scan_only"] = {"delta": -1e30, "keep_fraction": round(so["keep_fraction"], 5),
                            "us_per_step": round(so["us_per_step"], 3), "roofline_attend": roofline_of(so, None),
                            "layers_rotated": so["layers_rotated"]}
    if split:
        out["split_path"] = measure_split(w, delta, steps, warmup, c, d, torch, sm_scale, flush)
    if dense:
        dn = measure_dense(w, max(10, steps // 2), min(warmup, 5), d, torch, sm_scale, flush)
        out.update({"dense_us_per_step": round(dn["us_per_step"], 3), "dense_gbps": round(dn["gbps"], 1),
                    "dense_layers_rotated": dn["layers_rotated"],
                    "speedup_vs_dense": round(dn["us_per_step"] / r["us_per_step"], 3)})
    del c, d
    torch.cuda.empty_cache()
    return out


# run-time termination operating points (tau, phi, patience, stream blocks):
# from the bench's variant (loose) to settings that stop only once the running
# output has nearly stopped moving; 4-block streams give the 16K step as many
# work-groups as the union split (the default 16-block streams run 4x fewer)
ART_POINTS = ((0.05, 0.01, 1, 4), (0.02, 0.005, 2, 4), (0.01, 0.002, 2, 4), (0.005, 0.001, 3, 4),
              (0.005, 0.001, 3, 16))


def art_tradeoff(w, delta, steps, warmup, seed, torch, sm_scale, flush):
    """Run-time termination on workload `w`: per operating point the step time,
    the fraction of kept (query head, token) pairs actually folded in, and the
    output's error against full attention over K-hat (delta = +inf) beside the
    union step's own error at the same delta, so that a point can be chosen
    for an accuracy budget.  Same rotation and flush as every other leg."""
    import sparse_long_context_ffd_amd as ffd
    c, d = prepare(w, seed, torch)
    shape = ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len, sink=w.sink, local=w.local)
    base = ffd.PackedCache(shape)
    ffd.quantize_k(shape, d["k"], 0, w.max_len, base)
    ffd.pack_v(shape, d["v"], 0, w.max_len, base)
    ws = torch.empty(max([ffd.workspace_bytes(shape)] + [ffd.workspace_bytes_ex(shape, art=a) for a in ART_POINTS]),
                     dtype=torch.uint8, device="cuda")
    rows = (w.batch, w.q_heads, 128)
    full, ref = (torch.empty(rows, dtype=torch.float16, device="cuda") for _ in range(2))
    ffd.decode_attn(shape, d["q"], base, d["seq_lens"], math.inf, sm_scale, full, ws)
    ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, ref, ws)
    lens = d["seq_lens"].long()
    valid = torch.arange(w.max_len, device="cuda")[None, :] < lens[:, None]
    tok_total = int(lens.sum()) * w.kv_heads
    # kept (query head, token) pairs of the union step; termination only ever
    # folds in a subset of them.  The rotation is sized from the union step's
    # bytes, as for the other legs.
    tu = torch.zeros((w.batch, w.q_heads, w.max_len), dtype=torch.uint8, device="cuda")
    ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, ref, ws, debug={"tmask": tu})
    torch.cuda.synchronize()
    kept_pairs = ((tu == 1) & valid[:, None, :]).sum().item()
    del tu
    layer_bytes = sum(ffd.cache_bytes(shape).values())
    R = copies_for(SCAN_BYTES * tok_total + REFINE_BYTES * kept_pairs // w.group, layer_bytes)
    layers = [base] + [base.clone() for _ in range(R - 1)]

    def err(o):
        dd = o.float() - full.float()
        return round((dd.norm() / full.float().norm()).item(), 6)

    out = {"workload": w.name, "delta": delta, "union_rel_l2_vs_full": err(ref), "layers_rotated": R, "points": []}
    g = graph_of([lambda i=i: ffd.decode_attn(shape, d["q"], layers[i % R], d["seq_lens"], delta, sm_scale, ref,
                                              ws) for i in range(steps)], torch)
    g.replay()
    out["union_us_per_step"] = round(timed_replay(g, torch, flush) * 1e3 / steps, 3)
    del g
    for art in ART_POINTS:
        o = torch.empty(rows, dtype=torch.float16, device="cuda")
        tm = torch.zeros((w.batch, w.q_heads, w.max_len), dtype=torch.uint8, device="cuda")
        ffd.decode_attn(shape, d["q"], base, d["seq_lens"], delta, sm_scale, o, ws, debug={"tmask": tm}, art=art)
        torch.cuda.synchronize()
        folded = ((tm == 1) & valid[:, None, :]).sum().item()
        g = graph_of([lambda i=i: ffd.decode_attn(shape, d["q"], layers[i % R], d["seq_lens"], delta, sm_scale, o,
                                                  ws, art=art) for i in range(steps)], torch)
        g.replay()
        us = timed_replay(g, torch, flush) * 1e3 / steps
        del g
        out["points"].append({"tau_phi_patience_stream_blocks": list(art), "us_per_step": round(us, 3),
                              "folded_frac_of_kept": round(folded / max(kept_pairs, 1), 5),
                              "rel_l2_vs_full": err(o)})
    del layers, base, c, d
    torch.cuda.empty_cache()
    return out


def sweep_workload(L):
    """The Llama-8B-like decode layer (B=1, Hq=32, Hkv=8, delta 5) at context L,
    with the needle count of the 16K and 256K workloads' rule 16 * sqrt(L / 16K)."""
    from synthetic import Workload
    return Workload(f"llama8b_{L // 1024}k", 1, 32, 8, L, L, deltas=(5.0,),
                    needles=int(round(16 * math.sqrt(L / 16384))))


def slope(xs, ys):
    """Least-squares slope of ys over xs."""
    x, y = np.asarray(xs, float), np.asarray(ys, float)
    return float(np.polyfit(x, y, 1)[0])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, delta, c, sm_scale, budget_s=10.0):
    """The fp64 oracle (as it stands) on the host cores: one decode step of the
    whole workload (pack excluded), repeated until ~budget_s of CPU work."""
    from oracle import ffd_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    G = w.group
    packs = {(b, h): orc.quantize_k(c["k"][b, h]) for b in range(w.batch) for h in range(w.kv_heads)}
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        for (b, h), pk in packs.items():
            orc.decode_head(c["q"][b, h * G:(h + 1) * G], pk, c["v"][b, h], int(c["seq_lens"][b]), delta, sm_scale,
                            w.sink, w.local)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s and len(times) >= 3:
            break
    med = statistics.median(times)
    return {"value": med * 1e6, "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"numpy fp64 oracle decode step over all {w.batch * w.kv_heads} KV heads of {w.name} "
                      f"(delta={delta}, pack excluded), median of {len(times)} steps",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


LEGS = ("long", "qwen", "stress", "sweep", "art")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_16k")
    ap.add_argument("--delta", type=float, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help=f"comma-separated legs beside the headline (of {', '.join(LEGS)}; '' for none)")
    ap.add_argument("--no-long", action="store_true", help="skip every leg beside the headline")
    ap.add_argument("--no-variants", action="store_true", help="skip the selection-variant timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=256,
                    help="size of one plain device-to-device copy done before timing; profiles scale "
                         "the HBM byte counters by what they read for it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    legs = [] if args.no_long else [x for x in args.legs.split(",") if x]
    unknown = set(legs) - set(LEGS)
    if unknown:
        print(f"unknown legs {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import sparse_long_context_ffd_amd as ffd
    from synthetic import WORKLOADS
    ffd.lib()
    sm_scale = float(np.float32(1.0 / math.sqrt(128.0)))
    w = WORKLOADS[args.workload]
    delta = w.deltas[0] if args.delta is None else args.delta

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = Flush(torch)
    c, d = prepare(w, args.seed, torch)
    r = measure_ffd(w, delta, args.steps, args.warmup, c, d, torch, sm_scale, flush,
                    with_variants=not args.no_variants)
    dense = measure_dense(w, args.steps, args.warmup, d, torch, sm_scale, flush)
    achieved = r["attend_bytes"] / (r["attend_us_mean"] * 1e3)
    result = {
        "metric": METRIC,
        "value": round(r["us_per_step"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["us_per_step"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "seq_len": int(c["seq_lens"].max()), "delta": delta, "sink": w.sink, "local": w.local,
                   "head_dim": 128, "block": 64, "keep_fraction": round(r["keep_fraction"], 5),
                   "layers_rotated": r["layers_rotated"],
                   "read_between_visits_gb": round(r["read_between_visits"] / 1e9, 3),
                   "chunk_blocks": r["plan"][0]},
        "effective_gbps": round(r["step_bytes"] / (r["us_per_step"] * 1e3), 1),
        "kv_tokens_per_s": r["tokens"] / (r["us_per_step"] * 1e-6),  # KV token-heads (tokens x KV heads) per s
        "context_tokens_per_s": r["tokens"] / w.kv_heads / (r["us_per_step"] * 1e-6),  # sum_b L_b per s
        "us_per_step_spread": r["replay_spread"],
        "attend_kernel_us": round(r["attend_us_mean"], 3),
        "decode_loop_us_per_step": round(r["loop_us_per_step"], 3),
        "eager_us_per_step": round(r["eager_us_per_step"], 3),
        "cache_warm_us_per_step": round(r["cache_warm_us_per_step"], 3),
        "selection_variants": r["variants"],
        "dense_us_per_step": round(dense["us_per_step"], 3),
        "dense_layers_rotated": dense["layers_rotated"],
        "speedup_vs_dense": round(dense["us_per_step"] / r["us_per_step"], 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_bytes(w.name),
                     "kernel": "attend_kernel (fused Top-delta scan + refine" +
                               (", pseudo-max work-groups in the grid)" if r["pm_in_grid"] else ")"),
                     "bytes_per_launch": r["attend_bytes"], "kernel_sources": kernel_digest()},
    }
    del d
    torch.cuda.empty_cache()
    steps_leg = max(20, args.steps // 4)
    warm_leg = min(args.warmup, 10)
    if "long" in legs:
        result["long_context"] = leg("long_context", WORKLOADS["long_256k"], WORKLOADS["long_256k"].deltas[0],
                                     steps_leg, warm_leg, args.seed, torch, sm_scale, flush, scan_only=True,
                                     split=True)
    if "qwen" in legs:
        wq = WORKLOADS["qwen7b_b16_16k32k"]
        result["batched_qwen"] = leg("batched_qwen", wq, wq.deltas[0], steps_leg, warm_leg, args.seed, torch,
                                     sm_scale, flush)
    if "stress" in legs:
        wst = WORKLOADS["stress_b4_128k"]
        result["stress"] = leg("stress", wst, wst.deltas[0], steps_leg, warm_leg, args.seed, torch, sm_scale,
                               flush)
    if "sweep" in legs:
        pts = []
        for L in (16384, 32768, 65536, 131072, 262144):
            if L == 16384 and w.name == "llama8b_16k" and delta == 5.0:
                pt = {"seq_len": L, "us_per_step": result["value"], "keep_fraction": result["config"]["keep_fraction"],
                      "attend_kernel_us": result["attend_kernel_us"], "dense_us_per_step": result["dense_us_per_step"]}
            elif L == 262144 and "long_context" in result:
                lc = result["long_context"]
                pt = {"seq_len": L, "us_per_step": lc["us_per_step"], "keep_fraction": lc["keep_fraction"],
                      "attend_kernel_us": lc["roofline_attend"]["attend_kernel_us"],
                      "dense_us_per_step": lc["dense_us_per_step"]}
            else:
                x = leg("sweep", sweep_workload(L), 5.0, steps_leg, warm_leg, args.seed, torch, sm_scale, flush)
                pt = {"seq_len": L, "us_per_step": x["us_per_step"], "keep_fraction": x["keep_fraction"],
                      "attend_kernel_us": x["roofline_attend"]["attend_kernel_us"],
                      "dense_us_per_step": x["dense_us_per_step"]}
            pt["speedup_vs_dense"] = round(pt["dense_us_per_step"] / pt["us_per_step"], 3)
            pts.append(pt)
        xs = [p["seq_len"] / 1024 for p in pts]
        result["context_sweep"] = {
            "workload": "Llama-8B-like heads (B=1, Hq=32, Hkv=8, delta 5), 16 * sqrt(L / 16K) needles per KV head",
            "points": pts,
            "slope_us_per_1k_tokens": {"ffd": round(slope(xs, [p["us_per_step"] for p in pts]), 4),
                                       "dense": round(slope(xs, [p["dense_us_per_step"] for p in pts]), 4)}}

    if "art" in legs:
        result["art_tradeoff"] = [art_tradeoff(wa, wa.deltas[0], steps_leg, warm_leg, args.seed, torch, sm_scale,
                                               flush)
                                  for wa in (w, WORKLOADS["qwen7b_b16_16k32k"], WORKLOADS["stress_b4_128k"])]

    result["hbm_achievable"] = hbm_probe(torch)
    # the attend kernels' rates against the measured streaming-read rate too
    # (context beside `frac`, which stays against the nominal peak)
    rd = result["hbm_achievable"]["read_gbps"]
    result["roofline"]["frac_of_read_probe"] = round(result["roofline"]["achieved"] / rd, 4)
    for k in ("long_context", "batched_qwen", "stress"):
        if k in result:
            ra = result[k]["roofline_attend"]
            ra["frac_of_read_probe"] = round(ra["achieved"] / rd, 4)
            if "scan_only" in result[k]:
                so = result[k]["scan_only"]["roofline_attend"]
                so["frac_of_read_probe"] = round(so["achieved"] / rd, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w, delta, c, sm_scale)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
