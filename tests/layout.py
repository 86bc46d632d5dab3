"""Decode libffd's packed K-cache bytes into logical arrays (test helper).

Implements the byte layout documented in include/ffd.h, independently of the
HIP kernels and of the oracle, so packed bytes can be compared field by field
with ``oracle.ffd_oracle.quantize_k``.
"""
import numpy as np


def _code_maps():
    word = np.zeros((64, 128), np.int64)
    bit = np.zeros((64, 128), np.int64)
    for t in range(64):
        for ch in range(128):
            g, r = divmod(ch, 32)
            kq, j = divmod(r, 8)
            p = g // 2
            word[t, ch] = (t * 4 + kq) * 2 + p                      # 32-bit word index in the block
            d, odd = divmod(j, 2)
            if g % 2 == 0:
                bit[t, ch] = 24 + 2 * d if odd else 8 + 2 * d
            else:
                bit[t, ch] = 16 + 2 * d if odd else 2 * d
    return word, bit


def _sz_map():
    idx = np.zeros((64, 4), np.int64)
    for t in range(64):
        tt, kq, i = t // 16, (t // 4) % 4, t % 4
        for g in range(4):
            idx[t, g] = (((tt * 4 + g) * 4 + kq) * 16 + i * 4) // 2   # fp16 element index of the scale
    return idx


def _res_map():
    idx = np.zeros((64, 128), np.int64)
    for t in range(64):
        for ch in range(128):
            idx[t, ch] = ((ch // 16) * 64 + t) * 16 + ch % 16
    return idx


_WORD, _BIT = _code_maps()
_SZ = _sz_map()
_RES = _res_map()
_RSC = ((np.arange(64)[:, None] // 16) * 4 + np.arange(4)[None, :]) * 16 + np.arange(64)[:, None] % 16  # [t][g]


def _v_map(L_cap: int):
    """[t][ch] -> fp16 element index of the token-quad tiled V of one head."""
    t = np.arange(L_cap)[:, None]
    ch = np.arange(128)[None, :]
    return ((t // 4) * 128 + ch) * 4 + t % 4


def decode_v(v: np.ndarray, B: int, Hkv: int, L_cap: int) -> np.ndarray:
    """Tiled V bytes -> fp16 [B][Hkv][L_cap][128]."""
    return v.view(np.float16).reshape(B, Hkv, L_cap * 128)[..., _v_map(L_cap)]


def decode_cache(codes: np.ndarray, sz: np.ndarray, res: np.ndarray, rscale: np.ndarray,
                 B: int, Hkv: int, L_cap: int, v: np.ndarray = None):
    """Byte buffers (uint8, as copied from the GPU) -> dict of logical fields
    shaped like ``quantize_k`` output over [B][Hkv][L_cap] (plus "v" when the
    tiled V bytes are given)."""
    nb = L_cap // 64
    words = codes.view(np.uint32).reshape(B, Hkv, nb, 512)
    c = (words[..., _WORD] >> _BIT.astype(np.uint32)) & 3                     # [B,Hkv,nb,64,128]
    h = sz.view(np.float16).reshape(B, Hkv, nb, 512)
    scale = h[..., _SZ]
    zero = h[..., _SZ + 1]
    r = res.view(np.int8).reshape(B, Hkv, nb, 8192)[..., _RES]
    s8 = rscale.view(np.float16).reshape(B, Hkv, nb, 256)[..., _RSC]
    out = {} if v is None else {"v": decode_v(v, B, Hkv, L_cap)}
    return {
        **out,
        "codes": c.astype(np.uint8).reshape(B, Hkv, L_cap, 128),
        "scale": scale.reshape(B, Hkv, L_cap, 4),
        "zero": zero.reshape(B, Hkv, L_cap, 4),
        "res": r.reshape(B, Hkv, L_cap, 128),
        "rscale": s8.reshape(B, Hkv, L_cap, 4),
    }
