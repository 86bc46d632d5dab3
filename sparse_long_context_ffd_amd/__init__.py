"""FFD sparse decode attention for MI355X (gfx950): Python binding of libffd.

The compute runs in hand-written HIP kernels behind the C ABI declared in
``include/ffd.h``; this package only marshals PyTorch tensors into that ABI.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    FFDError,
    LIB_PATH,
    PackedCache,
    Shape,
    append_kv,
    cache_bytes,
    decode_attn,
    decode_attn_noalloc,
    dense_decode_attn,
    lib,
    make_shape,
    pack_v,
    plan,
    plan_pseudomax,
    plan_split,
    quantize_k,
    strerror,
    stream_read,
    workspace_bytes,
    workspace_bytes_ex,
)

__all__ = [
    "EXPORTED", "FFDError", "LIB_PATH", "PackedCache", "Shape", "append_kv", "cache_bytes", "decode_attn", "decode_attn_noalloc",
    "dense_decode_attn", "lib", "make_shape", "pack_v", "plan", "plan_pseudomax", "plan_split", "quantize_k", "strerror", "stream_read", "workspace_bytes",
    "workspace_bytes_ex",
]
