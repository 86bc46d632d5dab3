"""Shared helpers of the GPU parity tests: run libffd through its binding and
compare with the fp64 oracle by the parity rules.

Parity rules
------------
* packed codes, fp16 scale/zero, int8 residuals and fp16 residual scales:
  bit-exact;
* block mask: equal to the oracle's on every *pinned* block -- forced blocks,
  blocks where some head's oracle block max is >= its threshold + 1e-4, and
  blocks where every head's oracle block max is < its threshold - 1e-4;
  blocks within 1e-4 of a threshold are exempt (either choice is correct);
* attention output: compared with the oracle evaluated under the GPU's own
  mask: max |diff| <= 2e-3 and ||diff|| / ||ref|| <= 1e-3 (fp16 output).
"""
import math
import sys

import numpy as np

BAND = 1e-4
ATOL = 2e-3
RTOL_L2 = 1e-3
SM_SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def shape_for(w, chunk_blocks=0, sink=None, local=None):
    import sparse_long_context_ffd_amd as ffd
    return ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len,
                          sink=w.sink if sink is None else sink,
                          local=w.local if local is None else local, chunk_blocks=chunk_blocks)


def gpu_pack(shape, k_dev, v_dev=None, fill=0xFF, t_begin=0, t_end=None):
    """Pack K (and V, when given) tokens [t_begin, t_end) into a fresh cache
    whose bytes start as `fill`."""
    import sparse_long_context_ffd_amd as ffd
    cache = ffd.PackedCache(shape).fill_(fill)
    t_end = shape.max_seq_len if t_end is None else t_end
    ffd.quantize_k(shape, k_dev, t_begin, t_end, cache)
    if v_dev is not None:
        ffd.pack_v(shape, v_dev, t_begin, t_end, cache)
    return cache


def decode_cache_fields(cache, w):
    from tests.layout import decode_cache
    return decode_cache(**cache_to_host(cache), B=w.batch, Hkv=w.kv_heads, L_cap=w.max_len)


def cache_to_host(cache):
    return {f: getattr(cache, f).cpu().numpy() for f in ("codes", "sz", "res", "rscale", "v")}


def _decode_once(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws, select, art, pm_mode, split_mode=0):
    import sparse_long_context_ffd_amd as ffd
    B, Hq, Hkv = shape.batch, shape.num_q_heads, shape.num_kv_heads
    nb = shape.max_seq_len // 64
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    dbg = {
        "m_tilde": torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda"),
        "bmax": torch.full((B, Hq, nb), float("nan"), dtype=torch.float32, device="cuda"),
        "keep": torch.full((B, Hkv, nb), 7, dtype=torch.uint8, device="cuda"),
        "tmask": torch.full((B, Hq, shape.max_seq_len), 7, dtype=torch.uint8, device="cuda"),
    }
    ffd.decode_attn(shape, q_dev, cache, lens_dev, delta, sm_scale, out, ws,
                    debug={**dbg, "pm_mode": pm_mode, "split_mode": split_mode}, select=select, art=art)
    torch.cuda.synchronize()
    return {"out": out.float().cpu().numpy(), **{k: v.cpu().numpy() for k, v in dbg.items()}}


# the pseudo-max paths one decode is run through with the fused scan + refine
# kernel (debug pm_mode, in order, on one workspace zeroed before the first):
# inside the attend launch on the fresh workspace (no initialised sync words,
# so every chunk computes the pseudo-max itself), inside it again (the chunks
# read the words the leading work-groups publish), the separate launch, and
# inside it with every chunk forced to compute it.  Selection variants and
# run-time termination have the separate launch only.  A union step also runs
# the split scan + refine kernels (SPLIT: separate pseudo-max launch).
PM_PATHS = (2, 2, 1, 3)
SPLIT = (1, 2)


def ws_bytes(shape, select="union", art=None):
    """Workspace bytes for a decode call with these options."""
    import sparse_long_context_ffd_amd as ffd
    return max(ffd.workspace_bytes(shape), ffd.workspace_bytes_ex(shape, select, art))


def production_decode(shape, q_dev, cache, lens_dev, delta, torch, sm_scale=SM_SCALE, ws=None, select="union",
                      art=None):
    """The call as a user makes it (and as bench.py times it): no debug
    buffers, the library's own pseudo-max placement and launch split.
    Returns the fp16 output as float32 numpy."""
    import sparse_long_context_ffd_amd as ffd
    out = torch.full((shape.batch, shape.num_q_heads, 128), float("nan"), dtype=torch.float16, device="cuda")
    if ws is None:
        ws = torch.full((ws_bytes(shape, select, art),), 0x5A, dtype=torch.uint8, device="cuda")
    ffd.decode_attn(shape, q_dev, cache, lens_dev, delta, sm_scale, out, ws, select=select, art=art)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def gpu_decode(shape, q_dev, cache, lens_dev, delta, torch, sm_scale=SM_SCALE, ws=None, select="union", art=None):
    """One decode step through the C ABI.  Without a caller's workspace a
    union step runs through every pseudo-max path (PM_PATHS), which must agree
    bit for bit (same arithmetic, only the hand-over differs); the
    published-words run is returned.  The production call (no debug buffers,
    default placement) then runs twice on a fresh junk-filled workspace -- its
    first call on a workspace, then one that uses what the first published --
    and both outputs must equal the debug run's bit for bit, so every oracle
    comparison of the returned output also covers the production call."""
    import sparse_long_context_ffd_amd as ffd
    if ws is not None:
        return _decode_once(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws, select, art, 0)
    ws = torch.zeros(ws_bytes(shape, select, art), dtype=torch.uint8, device="cuda")
    if select != "union" or art is not None:
        got = _decode_once(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws, select, art, 0)
        prod = production_decode(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, select=select, art=art)
        assert np.array_equal(prod, got["out"]), f"production call ({select}, art={art}) differs from the debug run"
        return got
    runs = [_decode_once(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws, select, art, mode, 1)
            for mode in PM_PATHS]
    for mode, r in zip(PM_PATHS[1:], runs[1:]):
        for k, v in runs[0].items():
            assert np.array_equal(v, r[k], equal_nan=True), f"pseudo-max path (pm_mode {mode}) changed {k}"
    # the split scan + refine kernels: the same decisions and diagnostics bit
    # for bit (same arithmetic); the output differs only in summation order and
    # is held to the oracle separately (check_head, "out_split")
    sp = _decode_once(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws, select, art, *SPLIT)
    for k in ("m_tilde", "bmax", "keep", "tmask"):
        assert np.array_equal(sp[k], runs[1][k], equal_nan=True), f"split path changed {k}"
    got = dict(runs[1], out_split=sp["out"])
    split_default = ffd.plan_split(shape)
    pws = torch.full((ffd.workspace_bytes(shape),), 0x5A, dtype=torch.uint8, device="cuda")
    for i in range(2):
        prod = production_decode(shape, q_dev, cache, lens_dev, delta, torch, sm_scale, ws=pws)
        ref = sp["out"] if split_default else runs[1]["out"]
        assert np.array_equal(prod, ref), \
            f"production call {i} differs from the debug run of its path (split={split_default})"
    return got


def gpu_dense(shape, q_dev, k_dev, v_dev, lens_dev, torch, sm_scale=SM_SCALE, ws=None):
    import sparse_long_context_ffd_amd as ffd
    out = torch.empty((shape.batch, shape.num_q_heads, 128), dtype=torch.float16, device="cuda")
    if ws is None:
        ws = torch.empty(ffd.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    ffd.dense_decode_attn(shape, q_dev, k_dev, v_dev, lens_dev, sm_scale, out, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def mask_pins(o):
    """(pinned_keep, pinned_drop) boolean [nblk] from an oracle decode_head result."""
    bmax, thr = o["bmax"], o["thr"][:, None]
    pk = o["forced"] | (bmax >= thr + BAND).any(axis=0)
    pd = (~o["forced"]) & (bmax < thr - BAND).all(axis=0)
    return pk, pd


def check_head(orc, q16, pk_head, V16, L, delta, got, b, h, G, sink=64, local=256, sm_scale=SM_SCALE,
               label="", select="union"):
    """Compare one (b, kv head) of a GPU decode with the oracle; returns stats.

    The per-head token decisions of a selection variant (debug ``tmask``) must
    equal the oracle's wherever they are pinned -- support tokens, forced
    blocks, and estimates or block maxima farther than BAND from the head's
    threshold -- and the output is compared with the oracle evaluated under
    the GPU's block mask and token decisions."""
    nb = (L + 63) // 64
    o = orc.decode_head(q16, pk_head, V16, L, delta, sm_scale, sink, local)
    keep = got["keep"][b, h, :nb].astype(bool)
    assert set(np.unique(got["keep"][b, h, :nb]).tolist()) <= {0, 1}, f"{label} keep flags not 0/1"
    pk, pd = mask_pins(o)
    bad_keep = np.nonzero(pk & ~keep)[0]
    bad_drop = np.nonzero(pd & keep)[0]
    assert bad_keep.size == 0 and bad_drop.size == 0, \
        f"{label} mask mismatch on pinned blocks: missing {bad_keep[:10]}, extra {bad_drop[:10]}"
    mt = got["m_tilde"][b, h * G:(h + 1) * G]
    mt_err = float(np.abs(mt - o["m_tilde"]).max())
    bm = got["bmax"][b, h * G:(h + 1) * G, :nb]
    bm_err = float(np.abs(bm - o["bmax"]).max())
    assert mt_err <= BAND, f"{label} pseudo-max error {mt_err}"
    assert bm_err <= BAND, f"{label} block-max error {bm_err}"
    tmask = None
    if "tmask" in got:
        tok = np.repeat(keep, 64)[:L]
        tm = got["tmask"][b, h * G:(h + 1) * G, :L]
        assert set(np.unique(tm[:, tok]).tolist()) <= {0, 1}, f"{label} token flags not 0/1"
        want = orc.decode_head(q16, pk_head, V16, L, delta, sm_scale, sink, local, keep=keep,
                               select=select)["tmask"]
        thr = o["thr"][:, None]
        if select == "union":
            pinned = np.ones((G, L), bool)
        elif select == "head_block":
            pb = o["forced"][None, :] | (np.abs(o["bmax"] - thr) > BAND)
            pinned = np.repeat(pb, 64, axis=1)[:, :L]
        else:
            pinned = orc.support_mask(L, sink, local)[None, :] | (np.abs(o["s_est"] - thr) > BAND)
        pinned &= tok[None, :]
        bad = np.argwhere(pinned & ((tm == 1) != want))
        assert bad.size == 0, f"{label} {select}: token decisions differ at (head, token) {bad[:8].tolist()}"
        tmask = (tm == 1) & tok[None, :]
    ref = orc.decode_head(q16, pk_head, V16, L, delta, sm_scale, sink, local, keep=keep, tmask=tmask)["out"]
    for key in ("out", "out_split"):
        if key not in got:
            continue
        d = got[key][b, h * G:(h + 1) * G] - ref
        ma = float(np.abs(d).max())
        rl = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
        assert ma <= ATOL and rl <= RTOL_L2, f"{label} {key} max-abs {ma} rel-L2 {rl}"
        if key == "out":
            max_abs, rel, rmse = ma, rl, float(np.sqrt(np.mean(d * d)))
    return {"keep_frac": float(keep.mean()), "exempt": int(nb - pk.sum() - pd.sum()),
            "mt_err": mt_err, "bmax_err": bm_err, "max_abs": max_abs, "rel_l2": rel, "rmse": rmse,
            "mask_equal": bool((keep == o["keep"]).all()),
            "attended_frac": None if tmask is None else float(tmask.mean())}
