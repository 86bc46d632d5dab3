"""ctypes binding of libffd (include/ffd.h).  Argument marshalling only.

Every function forwards to the C entry point of the same name; tensors are
PyTorch tensors on the GPU and are passed as raw device pointers together with
the caller's current HIP stream.  There is no CPU fallback: if libffd.so is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffd.so")

FFD_OK = 0
STATUS = {
    0: "FFD_OK", -1: "FFD_ERR_NULL", -2: "FFD_ERR_SHAPE", -3: "FFD_ERR_ALIGN", -4: "FFD_ERR_DELTA",
    -5: "FFD_ERR_WORKSPACE", -6: "FFD_ERR_ARG", -7: "FFD_ERR_HIP", -8: "FFD_ERR_TOO_LARGE",
}
EXPORTED = (
    "ffd_cache_bytes", "ffd_workspace_bytes", "ffd_workspace_bytes_ex", "ffd_plan", "ffd_plan_pseudomax", "ffd_plan_split", "ffd_quantize_k", "ffd_pack_v", "ffd_append_kv",
    "ffd_decode_attn", "ffd_decode_attn_select", "ffd_decode_attn_ex", "ffd_decode_attn_noalloc",
    "ffd_dense_decode_attn", "ffd_stream_read", "ffd_strerror", "ffd_version",
)
STREAM_READ_SINK_BYTES = 8192  # FFD_STREAM_READ_SINK_BYTES
NOALLOC_SCRATCH_BYTES = 32 << 20  # FFD_NOALLOC_SCRATCH_BYTES


class FFDError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({strerror(code)})")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "block", "sink", "local",
        "max_seq_len", "chunk_blocks")]


class Cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("sz", ctypes.c_void_p), ("res", ctypes.c_void_p),
                ("rscale", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [("m_tilde", ctypes.c_void_p), ("bmax", ctypes.c_void_p), ("keep", ctypes.c_void_p),
                ("attend_start", ctypes.c_void_p), ("attend_stop", ctypes.c_void_p), ("stages", ctypes.c_int32),
                ("tmask", ctypes.c_void_p), ("pm_mode", ctypes.c_int32), ("split_mode", ctypes.c_int32)]

SELECTIONS = {"union": 0, "head_block": 1, "head_token": 2}


class DecodeOpts(ctypes.Structure):
    _fields_ = [("selection", ctypes.c_int32), ("art_patience", ctypes.c_int32), ("art_tau", ctypes.c_float),
                ("art_phi", ctypes.c_float), ("art_stream_blocks", ctypes.c_int32)]


ART_STREAM_BLOCKS_DEFAULT = 16  # FFD_ART_STREAM_BLOCKS_DEFAULT


_lib = None


def lib() -> ctypes.CDLL:
    """Load libffd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m sparse_long_context_ffd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, V, SZ, I32 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        L.ffd_cache_bytes.argtypes = [P(Shape), P(SZ), P(SZ), P(SZ), P(SZ), P(SZ)]
        L.ffd_workspace_bytes.argtypes = [P(Shape), P(SZ)]
        L.ffd_workspace_bytes_ex.argtypes = [P(Shape), P(DecodeOpts), P(SZ)]
        L.ffd_plan.argtypes = [P(Shape), P(I32), P(I32)]
        L.ffd_plan_pseudomax.argtypes = [P(Shape), P(I32), P(I32)]
        L.ffd_plan_split.argtypes = [P(Shape), P(I32)]
        L.ffd_quantize_k.argtypes = [P(Shape), V, I32, I32, P(Cache), V]
        L.ffd_pack_v.argtypes = [P(Shape), V, I32, I32, P(Cache), V]
        L.ffd_append_kv.argtypes = [P(Shape), V, V, V, P(Cache), V]
        L.ffd_decode_attn.argtypes = [P(Shape), V, P(Cache), V, ctypes.c_float, ctypes.c_float, V, V, SZ,
                                      P(Debug), V]
        L.ffd_decode_attn_select.argtypes = [P(Shape), V, P(Cache), V, ctypes.c_float, ctypes.c_float, I32, V,
                                             V, SZ, P(Debug), V]
        L.ffd_decode_attn_ex.argtypes = [P(Shape), V, P(Cache), V, ctypes.c_float, ctypes.c_float, P(DecodeOpts),
                                         V, V, SZ, P(Debug), V]
        L.ffd_decode_attn_noalloc.argtypes = [P(Shape), V, P(Cache), V, ctypes.c_float, ctypes.c_float, V, V]
        L.ffd_dense_decode_attn.argtypes = [P(Shape), V, V, V, V, ctypes.c_float, V, V, SZ, V]
        L.ffd_stream_read.argtypes = [V, SZ, V, V]
        L.ffd_strerror.argtypes = [ctypes.c_int]
        L.ffd_strerror.restype = ctypes.c_char_p
        L.ffd_version.argtypes = []
        for n in EXPORTED:
            if n not in ("ffd_strerror",):
                getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().ffd_strerror(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != FFD_OK:
        raise FFDError(code, where)


def make_shape(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int, sink: int = 64,
               local: int = 256, chunk_blocks: int = 0, head_dim: int = 128, block: int = 64) -> Shape:
    return Shape(batch, num_q_heads, num_kv_heads, head_dim, block, sink, local, max_seq_len, chunk_blocks)


FIELDS = ("codes", "sz", "res", "rscale", "v")


def cache_bytes(shape: Shape) -> dict:
    n = [ctypes.c_size_t() for _ in FIELDS]
    _check(lib().ffd_cache_bytes(ctypes.byref(shape), *(ctypes.byref(x) for x in n)), "ffd_cache_bytes")
    return {f: x.value for f, x in zip(FIELDS, n)}


def workspace_bytes(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(lib().ffd_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "ffd_workspace_bytes")
    return n.value


def _opts(select: str = "union", art=None) -> "DecodeOpts":
    if select not in SELECTIONS:
        raise ValueError(f"unknown selection {select!r}")
    if art is None:
        return DecodeOpts(SELECTIONS[select], 0, 0.0, 0.0, 0)
    tau, phi, patience = art[:3]
    stream_blocks = art[3] if len(art) > 3 else 0
    return DecodeOpts(SELECTIONS[select], int(patience), float(tau), float(phi), int(stream_blocks))


def workspace_bytes_ex(shape: Shape, select: str = "union", art=None) -> int:
    """Workspace bytes of one decode call with these options (``art`` as in
    decode_attn)."""
    n = ctypes.c_size_t()
    o = _opts(select, art)
    _check(lib().ffd_workspace_bytes_ex(ctypes.byref(shape), ctypes.byref(o), ctypes.byref(n)),
           "ffd_workspace_bytes_ex")
    return n.value


def plan(shape: Shape) -> Tuple[int, int]:
    cb, nc = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ffd_plan(ctypes.byref(shape), ctypes.byref(cb), ctypes.byref(nc)), "ffd_plan")
    return cb.value, nc.value


def plan_pseudomax(shape: Shape) -> Tuple[int, bool]:
    """(support parts per sequence, whether a whole union step runs the
    pseudo-max inside the scan + refine launch)."""
    n, g = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ffd_plan_pseudomax(ctypes.byref(shape), ctypes.byref(n), ctypes.byref(g)), "ffd_plan_pseudomax")
    return n.value, bool(g.value)


def plan_split(shape: Shape) -> bool:
    """Whether a whole union step runs stages 2 and 3 as the split scan +
    refine kernels (ffd_plan_split)."""
    n = ctypes.c_int32()
    _check(lib().ffd_plan_split(ctypes.byref(shape), ctypes.byref(n)), "ffd_plan_split")
    return bool(n.value)


# ---------------------------------------------------------------- tensor plumbing
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, dtype, numel, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name}: expected a contiguous {dtype} CUDA tensor with >= {numel} elements, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


class PackedCache:
    """Device buffers (uint8 tensors) of one layer's FFD cache: the packed K
    fields and the tiled fp16 V, layouts as in include/ffd.h."""

    def __init__(self, shape: Shape, device="cuda"):
        import torch
        nb = cache_bytes(shape)
        self.shape = shape
        for f in FIELDS:
            setattr(self, f, torch.empty(nb[f], dtype=torch.uint8, device=device))

    def fill_(self, byte: int) -> "PackedCache":
        for f in FIELDS:
            getattr(self, f).fill_(byte)
        return self

    def clone(self) -> "PackedCache":
        c = PackedCache.__new__(PackedCache)
        c.shape = self.shape
        for f in FIELDS:
            setattr(c, f, getattr(self, f).clone())
        return c

    def c_struct(self) -> Cache:
        return Cache(_ptr(self.codes), _ptr(self.sz), _ptr(self.res), _ptr(self.rscale), _ptr(self.v))


def quantize_k(shape: Shape, k, t_begin: int, t_end: int, cache: PackedCache, stream=None) -> None:
    import torch
    _need(k, torch.float16, shape.batch * shape.num_kv_heads * shape.max_seq_len * 128, "k")
    c = cache.c_struct()
    _check(lib().ffd_quantize_k(ctypes.byref(shape), _ptr(k), int(t_begin), int(t_end), ctypes.byref(c),
                                _stream(stream)), "ffd_quantize_k")


def pack_v(shape: Shape, v, t_begin: int, t_end: int, cache: PackedCache, stream=None) -> None:
    import torch
    _need(v, torch.float16, shape.batch * shape.num_kv_heads * shape.max_seq_len * 128, "v")
    c = cache.c_struct()
    _check(lib().ffd_pack_v(ctypes.byref(shape), _ptr(v), int(t_begin), int(t_end), ctypes.byref(c),
                            _stream(stream)), "ffd_pack_v")


def append_kv(shape: Shape, k_new, v_new, pos, cache: PackedCache, stream=None) -> None:
    """Write one token per sequence at the device positions ``pos`` (int32 [B])."""
    import torch
    n = shape.batch * shape.num_kv_heads * 128
    _need(k_new, torch.float16, n, "k_new")
    _need(v_new, torch.float16, n, "v_new")
    _need(pos, torch.int32, shape.batch, "pos")
    nb = cache_bytes(shape)
    for f in FIELDS:
        _need(getattr(cache, f), torch.uint8, nb[f], f"cache.{f}")
    c = cache.c_struct()
    _check(lib().ffd_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(pos), ctypes.byref(c),
                               _stream(stream)), "ffd_append_kv")


def decode_attn(shape: Shape, q, cache: PackedCache, seq_lens, delta: float, sm_scale: float, out,
                workspace, debug: Optional[dict] = None, stream=None, select: str = "union",
                art: Optional[Tuple[float, float, int]] = None) -> None:
    """One decode step; ``select`` is "union" (ffd_decode_attn) or a selection
    variant "head_block" / "head_token" (ffd_decode_attn_select); ``art`` =
    (tau, phi, patience[, stream_blocks]) turns on the run-time termination
    of each refine stream (ffd_decode_attn_ex; stream_blocks 0 or absent =
    the default length)."""
    import torch
    rows = shape.batch * shape.num_q_heads
    _need(q, torch.float16, rows * 128, "q")
    _need(out, torch.float16, rows * 128, "out")
    _need(seq_lens, torch.int32, shape.batch, "seq_lens")
    nb = cache_bytes(shape)
    for f in FIELDS:
        _need(getattr(cache, f), torch.uint8, nb[f], f"cache.{f}")
    _need(workspace, torch.uint8, 0, "workspace")
    c = cache.c_struct()
    dbg = None
    if debug is not None:
        dbg = Debug(_ptr(debug.get("m_tilde")), _ptr(debug.get("bmax")), _ptr(debug.get("keep")),
                    debug.get("attend_start"), debug.get("attend_stop"), int(debug.get("stages", 0)),
                    _ptr(debug.get("tmask")), int(debug.get("pm_mode", 0)), int(debug.get("split_mode", 0)))
    if art is not None:
        opts = _opts(select, art)
        _check(lib().ffd_decode_attn_ex(ctypes.byref(shape), _ptr(q), ctypes.byref(c), _ptr(seq_lens),
                                        float(delta), float(sm_scale), ctypes.byref(opts), _ptr(out),
                                        _ptr(workspace), workspace.numel(),
                                        None if dbg is None else ctypes.byref(dbg), _stream(stream)),
               "ffd_decode_attn_ex")
    elif select == "union":
        _check(lib().ffd_decode_attn(ctypes.byref(shape), _ptr(q), ctypes.byref(c), _ptr(seq_lens),
                                     float(delta), float(sm_scale), _ptr(out), _ptr(workspace),
                                     workspace.numel(), None if dbg is None else ctypes.byref(dbg),
                                     _stream(stream)), "ffd_decode_attn")
    else:
        if select not in SELECTIONS:
            raise ValueError(f"unknown selection {select!r}")
        _check(lib().ffd_decode_attn_select(ctypes.byref(shape), _ptr(q), ctypes.byref(c), _ptr(seq_lens),
                                            float(delta), float(sm_scale), SELECTIONS[select], _ptr(out),
                                            _ptr(workspace), workspace.numel(),
                                            None if dbg is None else ctypes.byref(dbg), _stream(stream)),
               "ffd_decode_attn_select")


def decode_attn_noalloc(shape: Shape, q, cache: PackedCache, seq_lens, delta: float, sm_scale: float, out,
                        stream=None) -> None:
    """ffd_decode_attn_noalloc: one union decode step whose workspace is the
    library's static per-GPU scratch array (no allocation by the call)."""
    import torch
    rows = shape.batch * shape.num_q_heads
    _need(q, torch.float16, rows * 128, "q")
    _need(out, torch.float16, rows * 128, "out")
    _need(seq_lens, torch.int32, shape.batch, "seq_lens")
    nb = cache_bytes(shape)
    for f in FIELDS:
        _need(getattr(cache, f), torch.uint8, nb[f], f"cache.{f}")
    c = cache.c_struct()
    _check(lib().ffd_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), ctypes.byref(c), _ptr(seq_lens),
                                         float(delta), float(sm_scale), _ptr(out), _stream(stream)),
           "ffd_decode_attn_noalloc")


def dense_decode_attn(shape: Shape, q, k, v, seq_lens, sm_scale: float, out, workspace, stream=None) -> None:
    import torch
    rows = shape.batch * shape.num_q_heads
    n = shape.batch * shape.num_kv_heads * shape.max_seq_len * 128
    _need(q, torch.float16, rows * 128, "q")
    _need(out, torch.float16, rows * 128, "out")
    _need(k, torch.float16, n, "k")
    _need(v, torch.float16, n, "v")
    _need(seq_lens, torch.int32, shape.batch, "seq_lens")
    _need(workspace, torch.uint8, 0, "workspace")
    _check(lib().ffd_dense_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens),
                                       float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                       _stream(stream)), "ffd_dense_decode_attn")


def stream_read(src, sink, stream=None) -> None:
    """Streaming-read probe (a measurement aid, not part of the decode path):
    reads every byte of the device tensor `src` once; `sink` (uint8 device
    tensor of STREAM_READ_SINK_BYTES) receives one 32-bit XOR per work-group."""
    import torch
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    _need(sink, torch.uint8, STREAM_READ_SINK_BYTES, "sink")
    _check(lib().ffd_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "ffd_stream_read")
