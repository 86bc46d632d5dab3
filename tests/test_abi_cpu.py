"""C-ABI checks that need no GPU: exports, argument validation, planning, layout maps.

Every call here fails validation (or is a pure host query) before any HIP
call, so nothing touches a device.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import sparse_long_context_ffd_amd as ffd
from sparse_long_context_ffd_amd import _lib
from tests import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ffd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    L = ffd.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.ffd_version() == 800


def test_strerror_covers_codes():
    for code in range(0, -9, -1):
        assert "unknown" not in ffd.strerror(code)
    assert "unknown" in ffd.strerror(-99)


FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation first


def _ws(shape):
    return ffd.workspace_bytes(shape)


def _decode(shape, q=FAKE, cache=None, lens=FAKE, delta=5.0, scale=0.088, out=FAKE, ws=FAKE, wsb=None):
    c = cache or _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    return ffd.lib().ffd_decode_attn(None if shape is None else ctypes.byref(shape), q, ctypes.byref(c), lens,
                                     delta, scale, out, ws, _ws(shape) if wsb is None else wsb, None, None)


def test_shape_validation():
    good = ffd.make_shape(1, 32, 8, 16384)
    assert ffd.workspace_bytes(good) > 0
    bad = [
        dict(head_dim=64), dict(block=32), dict(num_q_heads=30), dict(num_q_heads=72),  # G = 9
        dict(max_seq_len=1000), dict(max_seq_len=0), dict(sink=-1), dict(local=-1),
        dict(sink=0, local=0), dict(chunk_blocks=-2), dict(batch=0), dict(num_kv_heads=0),
        dict(batch=65536), dict(num_q_heads=65536, num_kv_heads=65536),  # grid dimensions
        dict(max_seq_len=1 << 24), dict(max_seq_len=(1 << 24) + 64),      # 32-bit block offsets
    ]
    for kw in bad:
        args = dict(batch=1, num_q_heads=32, num_kv_heads=8, max_seq_len=16384)
        args.update(kw)
        s = ffd.make_shape(**{k: v for k, v in args.items() if k in ("batch", "num_q_heads", "num_kv_heads",
                                                                     "max_seq_len", "sink", "local",
                                                                     "chunk_blocks", "head_dim", "block")})
        n = ctypes.c_size_t()
        assert ffd.lib().ffd_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == -2, kw
        assert _decode(s, wsb=1 << 30) == -2, kw
    assert ffd.lib().ffd_workspace_bytes(None, ctypes.byref(ctypes.c_size_t())) == -1
    # the longest cache the 32-bit offsets address
    assert ffd.workspace_bytes(ffd.make_shape(1, 4, 1, (1 << 24) - 64)) > 0


def test_decode_argument_errors():
    s = ffd.make_shape(1, 32, 8, 16384)
    assert _decode(s, q=None) == -1
    assert _decode(s, out=None) == -1
    assert _decode(s, lens=None) == -1
    assert _decode(s, cache=_lib.Cache(FAKE, FAKE, FAKE, FAKE, None)) == -1
    assert _decode(s, q=FAKE + 8) == -3
    assert _decode(s, cache=_lib.Cache(FAKE, FAKE + 4, FAKE, FAKE, FAKE)) == -3
    assert _decode(s, lens=FAKE + 2) == -3
    assert _decode(s, delta=math.nan) == -4
    assert _decode(s, delta=-math.inf) == -4
    assert _decode(s, scale=0.0) == -6
    assert _decode(s, scale=-1.0) == -6
    assert _decode(s, scale=math.inf) == -6
    assert _decode(s, scale=math.nan) == -6
    assert _decode(s, wsb=_ws(s) - 1) == -5
    assert _decode(s, ws=None) == -5
    assert _decode(s, ws=FAKE + 8) == -3


def test_debug_argument_errors():
    """Debug stage masks and pseudo-max modes are validated before any launch."""
    s = ffd.make_shape(1, 32, 8, 16384)
    c = _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)

    def dec(stages, pm_mode, shape=s, selection=0, art=0, split_mode=0):
        d = _lib.Debug(None, None, None, None, None, stages, None, pm_mode, split_mode)
        o = _lib.DecodeOpts(selection, art, 0.1, 0.1)
        return ffd.lib().ffd_decode_attn_ex(ctypes.byref(shape), FAKE, ctypes.byref(c), FAKE, 5.0, 0.088,
                                            ctypes.byref(o), FAKE, FAKE, _ws(shape), ctypes.byref(d), None)
    assert dec(32, 0) == -6 and dec(-1, 0) == -6
    assert dec(0, 4) == -6 and dec(0, -1) == -6
    # the pseudo-max inside the attend launch needs the merge in the same call,
    for mode in (2, 3):
        for stages in (1, 2, 3, 4, 5):
            assert dec(stages, mode) == -6, (stages, mode)
        # the union selection without run-time termination,
        assert dec(0, mode, selection=1) == -6 and dec(0, mode, selection=2) == -6
        assert dec(0, mode, art=2) == -6
        # and the support words of a work-group (npart * G <= 256)
        big = ffd.make_shape(1, 8, 1, 1 << 20, local=(1 << 20) - 64)
        assert dec(0, mode, shape=big) == -6
    # split path: modes 0..2; forcing it needs the union selection, no run-time
    # termination and the pseudo-max in its own launch; the scan / refine stage
    # bits exist on it only (16K runs fused by default, 256K split)
    assert dec(0, 1, split_mode=3) == -6 and dec(0, 1, split_mode=-1) == -6
    assert dec(0, 2, split_mode=2) == -6 and dec(0, 3, split_mode=2) == -6
    assert dec(0, 1, split_mode=2, selection=1) == -6 and dec(0, 1, split_mode=2, art=2) == -6
    for st in (8, 16, 24):
        assert dec(st, 0) == -6 and dec(st, 1, split_mode=1) == -6
    long_ = ffd.make_shape(1, 32, 8, 262144)
    assert not ffd.plan_split(s) and not ffd.plan_split(long_)  # the fused kernel is the default
    assert dec(8, 0, shape=long_, split_mode=1) == -6 and dec(16, 0, shape=long_) == -6
    # too many bitmap words for the refine's LDS: no split path
    wide = ffd.make_shape(64, 64, 8, 262144)
    assert dec(0, 1, shape=wide, split_mode=2) == -6


def _decode_sel(shape, selection, q=FAKE, ws=FAKE):
    c = _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    return ffd.lib().ffd_decode_attn_select(ctypes.byref(shape), q, ctypes.byref(c), FAKE, 5.0, 0.088, selection,
                                            FAKE, ws, _ws(shape), None, None)


def test_decode_select_argument_errors():
    s = ffd.make_shape(1, 32, 8, 16384)
    for bad in (-1, 3, 7, 1 << 20):
        assert _decode_sel(s, bad) == -6, bad
    for sel in (0, 1, 2):                       # valid codes still validate the rest first
        assert _decode_sel(s, sel, q=None) == -1
        assert _decode_sel(s, sel, ws=FAKE + 8) == -3
    assert set(_lib.SELECTIONS.values()) == {0, 1, 2}


def _decode_ex(shape, opts, q=FAKE, wsb=None):
    c = _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    return ffd.lib().ffd_decode_attn_ex(ctypes.byref(shape), q, ctypes.byref(c), FAKE, 5.0, 0.088,
                                        None if opts is None else ctypes.byref(opts), FAKE, FAKE,
                                        _ws(shape) if wsb is None else wsb, None, None)


def test_decode_ex_option_errors():
    s = ffd.make_shape(1, 32, 8, 16384)
    O = _lib.DecodeOpts
    for bad in (O(3, 0, 0.0, 0.0), O(0, -1, 0.0, 0.0), O(1, 2, 0.1, 0.1), O(2, 1, 0.1, 0.1),
                O(0, 1, -0.1, 0.1), O(0, 1, 0.1, math.nan), O(0, 1, math.inf, 0.1), O(0, 1, 0.1, -math.inf)):
        assert _decode_ex(s, bad) == -6, (bad.selection, bad.art_patience, bad.art_tau, bad.art_phi)
    for good in (None, O(0, 0, 0.0, 0.0), O(0, 2, 0.05, 0.01), O(2, 0, -1.0, math.nan)):
        assert _decode_ex(s, good, q=None) == -1       # valid options: the pointer checks still run first


def test_art_stream_length_and_workspace():
    """The run-time termination stream length is validated per group size and
    sizes the workspace of the call (ffd_workspace_bytes_ex)."""
    O = _lib.DecodeOpts
    s4 = ffd.make_shape(1, 32, 8, 16384)        # G = 4: up to 32 blocks per stream
    s8 = ffd.make_shape(1, 64, 8, 16384)        # G = 8: up to 16
    for sh, bad in ((s4, 33), (s4, -1), (s8, 17)):
        assert _decode_ex(sh, O(0, 1, 0.1, 0.1, bad), wsb=1 << 30) == -6, bad
        n = ctypes.c_size_t()
        assert ffd.lib().ffd_workspace_bytes_ex(ctypes.byref(sh), ctypes.byref(O(0, 1, 0.1, 0.1, bad)),
                                                ctypes.byref(n)) == -6
    for sh, good in ((s4, 32), (s4, 1), (s8, 16), (s8, 0)):
        assert _decode_ex(sh, O(0, 1, 0.1, 0.1, good), q=None) == -1
    # partials: one per stream; the default length fits ffd_workspace_bytes, a
    # 1-block stream on a 256K cache needs more
    assert ffd.workspace_bytes_ex(s4, art=(0.1, 0.1, 1)) <= ffd.workspace_bytes(s4)
    s4l = ffd.make_shape(1, 32, 8, 262144)
    rows, nblk = 32, 262144 // 64
    assert ffd.workspace_bytes_ex(s4l, art=(0.1, 0.1, 1)) <= ffd.workspace_bytes(s4l)
    one = ffd.workspace_bytes_ex(s4l, art=(0.1, 0.1, 1, 1))
    assert one >= rows * nblk * (128 + 2) * 4 > ffd.workspace_bytes(s4l)
    # the stream length is ignored without termination; opts NULL = the plain step
    assert ffd.workspace_bytes_ex(s4) == ffd.workspace_bytes_ex(s4, art=None)
    n = ctypes.c_size_t()
    assert ffd.lib().ffd_workspace_bytes_ex(ctypes.byref(s4), None, ctypes.byref(n)) == 0
    assert n.value == ffd.workspace_bytes_ex(s4) <= ffd.workspace_bytes(s4)
    # a call with a too-small workspace for its stream length is refused
    assert _decode_ex(s4l, O(0, 1, 0.1, 0.1, 1), wsb=ffd.workspace_bytes(s4l)) == -5
    assert _decode_ex(s4l, O(0, 1, 0.1, 0.1, 1), q=None, wsb=one) == -1


def test_dense_and_pack_argument_errors():
    s = ffd.make_shape(2, 8, 2, 4096)
    L = ffd.lib()
    wsb = _ws(s)
    assert L.ffd_dense_decode_attn(ctypes.byref(s), FAKE, None, FAKE, FAKE, 0.1, FAKE, FAKE, wsb, None) == -1
    assert L.ffd_dense_decode_attn(ctypes.byref(s), FAKE, FAKE + 2, FAKE, FAKE, 0.1, FAKE, FAKE, wsb, None) == -3
    assert L.ffd_dense_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE, wsb, None) == -6
    assert L.ffd_dense_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, wsb - 1, None) == -5
    c = _lib.Cache(FAKE, FAKE, FAKE, FAKE, None)
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE, -1, 5, ctypes.byref(c), None) == -6
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE, 6, 5, ctypes.byref(c), None) == -6
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE, 0, 4097, ctypes.byref(c), None) == -6
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE, 10, 10, ctypes.byref(c), None) == 0   # empty range: no-op
    assert L.ffd_quantize_k(ctypes.byref(s), None, 0, 5, ctypes.byref(c), None) == -1
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE + 6, 0, 5, ctypes.byref(c), None) == -3
    assert L.ffd_quantize_k(ctypes.byref(s), FAKE, 0, 5, ctypes.byref(_lib.Cache(FAKE, None, FAKE, FAKE, None)),
                            None) == -1
    cv = _lib.Cache(None, None, None, None, FAKE)      # ffd_pack_v reads only cache->v
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, -1, 5, ctypes.byref(cv), None) == -6
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, 6, 5, ctypes.byref(cv), None) == -6
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, 0, 4097, ctypes.byref(cv), None) == -6
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, 7, 7, ctypes.byref(cv), None) == 0
    assert L.ffd_pack_v(ctypes.byref(s), None, 0, 5, ctypes.byref(cv), None) == -1
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, 0, 5, ctypes.byref(_lib.Cache(FAKE, FAKE, FAKE, FAKE, None)),
                        None) == -1
    assert L.ffd_pack_v(ctypes.byref(s), FAKE + 2, 0, 5, ctypes.byref(cv), None) == -3
    assert L.ffd_pack_v(ctypes.byref(s), FAKE, 0, 5, ctypes.byref(_lib.Cache(None, None, None, None, FAKE + 8)),
                        None) == -3
    full = _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.ffd_append_kv(ctypes.byref(s), None, FAKE, FAKE, ctypes.byref(full), None) == -1
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, None, FAKE, ctypes.byref(full), None) == -1
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, FAKE, None, ctypes.byref(full), None) == -1
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(c), None) == -1     # cache->v NULL
    assert L.ffd_append_kv(ctypes.byref(s), FAKE + 2, FAKE, FAKE, ctypes.byref(full), None) == -3
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, FAKE + 8, FAKE, ctypes.byref(full), None) == -3
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, FAKE, FAKE + 2, ctypes.byref(full), None) == -3
    assert L.ffd_append_kv(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(_lib.Cache(FAKE, FAKE, FAKE + 4, FAKE,
                                                                                      FAKE)), None) == -3
    bad = _lib.Shape(1, 4, 1, 64, 64, 64, 256, 4096, 0)
    assert L.ffd_append_kv(ctypes.byref(bad), FAKE, FAKE, FAKE, ctypes.byref(full), None) == -2


def test_cache_and_workspace_sizes():
    s = ffd.make_shape(2, 28, 4, 32768)
    nb = ffd.cache_bytes(s)
    blocks = 2 * 4 * 512
    assert nb == {"codes": blocks * 2048, "sz": blocks * 1024, "res": blocks * 8192, "rscale": blocks * 512,
                  "v": blocks * 16384}
    per_token = sum(nb.values()) / (2 * 4 * 32768)
    # 2-bit codes 32 + (scale, zero) 16 + int8 residual 128 + rscale 8 + fp16 V 256
    assert per_token == 440
    cb, nch = ffd.plan(s)
    assert nch == math.ceil(512 / cb)
    rows = 2 * 28
    npart = 1 + 4 + 1                 # sink block, blocks of the local window, one straddling block
    # sync words (16 B), in-grid pseudo-max words (8 B), separate-launch maxima
    # (4 B), chunk (m, l) and o partials; each region 256-byte aligned
    need = 16 + rows * npart * 8 + rows * npart * 4 + rows * nch * 8 + rows * nch * 128 * 4
    # the split path instead: keep bitmap words, unit starts, and a partial per
    # refine unit and query head of the group (at most 2048 + B*Hkv units)
    heads, G = 2 * 4, 7
    need_split = (16 + rows * npart * 8 + rows * npart * 4 + heads * math.ceil(512 / 32) * 4 + (heads + 1) * 4
                  + (2048 + heads) * G * (8 + 128 * 4))
    need = max(need, need_split)
    assert need <= ffd.workspace_bytes(s) <= need + 8 * 256


def test_workspace_covers_the_dense_and_split_paths():
    # at 256K the fused decode splits into 24-block chunks, the dense baseline
    # into 16-block ones, the split path into refine units: the workspace holds
    # the largest set of partials
    s = ffd.make_shape(1, 32, 8, 262144)
    assert ffd.plan(s)[0] == 24
    rows, npart, nch_dense, heads, G = 32, 6, 4096 // 16, 8, 4
    head = 16 + rows * npart * 8 + rows * npart * 4
    need_dense = head + rows * nch_dense * (8 + 128 * 4)
    need_split = head + heads * (4096 // 32) * 4 + (heads + 1) * 4 + (2048 + heads) * G * (8 + 128 * 4)
    need = max(need_dense, need_split)
    assert need <= ffd.workspace_bytes(s) <= need + 8 * 256


@pytest.mark.parametrize("B,Hq,Hkv,L", [(1, 32, 8, 16384), (1, 4, 1, 4096), (1, 32, 8, 262144),
                                         (16, 28, 4, 32768), (4, 32, 8, 131072)])
def test_plan_pseudomax(B, Hq, Hkv, L):
    """Support parts (sink block, local-window blocks, one straddling block) and
    the pseudo-max's placement: inside the scan + refine launch whenever the
    support words fit one per thread of a work-group."""
    s = ffd.make_shape(B, Hq, Hkv, L)
    n, g = ffd.plan_pseudomax(s)
    assert n == 1 + 4 + 1 and g is True
    out = ctypes.c_int32()
    assert ffd.lib().ffd_plan_pseudomax(ctypes.byref(s), None, ctypes.byref(out)) == -1
    assert ffd.lib().ffd_plan_pseudomax(ctypes.byref(s), ctypes.byref(out), None) == -1
    bad = ffd.make_shape(B, Hq, Hkv, L)
    bad.head_dim = 64
    assert ffd.lib().ffd_plan_pseudomax(ctypes.byref(bad), ctypes.byref(out), ctypes.byref(out)) == -2
    # a local window wider than 256 query heads' worth of words keeps its own launch
    wide = ffd.make_shape(1, 8, 1, 1 << 20, local=(1 << 20) - 64)
    assert ffd.plan_pseudomax(wide)[1] is False


@pytest.mark.parametrize("B,Hq,Hkv,L,expect", [(1, 32, 8, 16384, 4), (1, 32, 8, 262144, 24),
                                               (16, 28, 4, 32768, 24), (1, 4, 1, 4096, 1),
                                               (4, 32, 8, 131072, 32), (1, 1, 1, 64, 1)])
def test_automatic_split(B, Hq, Hkv, L, expect):
    """About 1380 work-groups per launch on long caches, up to 4 blocks per work-group on
    short ones; at most 32 blocks per chunk (24 when G > 4)."""
    cb, nch = ffd.plan(ffd.make_shape(B, Hq, Hkv, L))
    assert cb == expect and nch == math.ceil(L // 64 / cb)
    cb, nch = ffd.plan(ffd.make_shape(B, Hq, Hkv, L, chunk_blocks=10 ** 6))
    cap = 32 if Hq // Hkv <= 4 else 24
    assert cb == min(cap, L // 64) and nch == math.ceil(L // 64 / cb)


def test_layout_maps_are_bijective():
    """Each code bit, (scale, zero) slot and residual byte of a block is used exactly once."""
    bits = layout._WORD * 32 + layout._BIT
    assert np.unique(np.concatenate([bits.ravel(), bits.ravel() + 1])).size == 64 * 128 * 2
    assert (layout._BIT % 2 == 0).all() and layout._WORD.max() == 511
    sz = layout._SZ
    assert np.unique(np.concatenate([sz.ravel(), sz.ravel() + 1])).size == 512
    assert np.unique(layout._RES).size == 8192 and layout._RES.max() == 8191
    assert np.unique(layout._RSC).size == 256


def test_stream_read_argument_errors():
    L = ffd.lib()
    assert L.ffd_stream_read(None, 16, FAKE, None) == -1
    assert L.ffd_stream_read(FAKE, 16, None, None) == -1
    assert L.ffd_stream_read(FAKE + 8, 16, FAKE, None) == -3   # src not 16-byte aligned
    assert L.ffd_stream_read(FAKE, 24, FAKE, None) == -3       # not a whole number of 16-byte words
    assert L.ffd_stream_read(FAKE, 16, FAKE + 2, None) == -3   # sink not 4-byte aligned
    assert _lib.STREAM_READ_SINK_BYTES == 8192
    text = open(HEADER).read()
    assert re.search(r"#define FFD_STREAM_READ_SINK_BYTES 8192\b", text)


def _noalloc(shape, q=FAKE, cache=None, lens=FAKE, delta=5.0, scale=0.088, out=FAKE):
    c = cache or _lib.Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    return ffd.lib().ffd_decode_attn_noalloc(None if shape is None else ctypes.byref(shape), q, ctypes.byref(c),
                                             lens, delta, scale, out, None)


def test_noalloc_argument_errors():
    """The allocation-free step validates like ffd_decode_attn, and a shape whose
    workspace exceeds the static scratch array is refused before any HIP call."""
    s = ffd.make_shape(1, 32, 8, 16384)
    assert _noalloc(None) == -1
    assert _noalloc(s, q=None) == -1
    assert _noalloc(s, out=None) == -1
    assert _noalloc(s, lens=None) == -1
    assert _noalloc(s, q=FAKE + 8) == -3
    assert _noalloc(s, delta=float("nan")) == -4
    assert _noalloc(s, scale=0.0) == -6
    assert _noalloc(ffd.make_shape(1, 32, 8, 1000)) == -2
    big = ffd.make_shape(64, 64, 8, 262144)
    assert ffd.workspace_bytes(big) > _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == -8
    assert "FFD_NOALLOC_SCRATCH_BYTES" in ffd.strerror(-8)
    # the header's size is the binding's
    text = open(HEADER).read()
    assert re.search(r"#define FFD_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)
    assert _lib.NOALLOC_SCRATCH_BYTES == 32 << 20
    # every workload of the benchmark fits
    from synthetic import WORKLOADS
    for w in WORKLOADS.values():
        sw = ffd.make_shape(w.batch, w.q_heads, w.kv_heads, w.max_len, sink=w.sink, local=w.local)
        assert ffd.workspace_bytes(sw) <= _lib.NOALLOC_SCRATCH_BYTES, w.name
