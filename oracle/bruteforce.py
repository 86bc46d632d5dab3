"""Naive exact-arithmetic FFD reference for tiny inputs (test infrastructure only).

Written independently of ``ffd_oracle``: pure Python loops, every quantizer
decision taken on ``fractions.Fraction`` values, rounding to fp16 done from
the exact rational by hand, dot products summed exactly.  It follows the same
page ("Faster Than Flash", gist.science summary of arXiv 2609.00097; Method
sections 1-3) and the same readings as ``ffd_oracle``; its only purpose is to
pin ``ffd_oracle`` on small cases.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Sequence

HALF = Fraction(1, 2)
F16_MAX = Fraction(65504)


def rne_binary16(x: Fraction) -> Fraction:
    """Round a rational to IEEE binary16, nearest with ties to even (finite range only)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                     # below 2^-14 the spacing stays 2^-24 (subnormals)
    ulp = Fraction(2) ** (e - 10)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > HALF or (rem == HALF and n % 2 == 1):
        n += 1
    r = n * ulp
    if r > F16_MAX:
        raise OverflowError("value outside the finite fp16 range")
    return sign * r


def pack_group(xs: Sequence[float]) -> Dict[str, object]:
    """Quantize one 32-value group of fp16 numbers (given as Python floats)."""
    X = [Fraction(x) for x in xs]
    z = min(X)
    s = rne_binary16((max(X) - z) / 3)
    codes = []
    for x in X:
        c = 0
        if s != 0:
            for k in (1, 2, 3):
                if x - z >= (k - HALF) * s:
                    c += 1
        codes.append(c)
    deq = [z + c * s for c in codes]
    r = [x - d for x, d in zip(X, deq)]
    s8 = rne_binary16(max(abs(v) for v in r) / 127)
    res = []
    for v in r:
        if s8 == 0:
            res.append(0)
            continue
        # #{j >= 1 : |v| >= (j - 1/2) s8} is the largest j with j <= |v|/s8 + 1/2 (exact rational floor)
        k = min(math.floor(abs(v) / s8 + HALF), 127)
        res.append(k if v > 0 else (-k if v < 0 else 0))
    khat = [d + e * s8 for d, e in zip(deq, res)]
    return {"codes": codes, "scale": s, "zero": z, "res": res, "rscale": s8,
            "deq2": deq, "khat": khat}


def pack_token(k: Sequence[float]) -> Dict[str, List]:
    """Quantize one 128-channel key (4 groups of 32)."""
    gs = [pack_group(k[32 * g: 32 * g + 32]) for g in range(4)]
    return {
        "codes": sum((g["codes"] for g in gs), []),
        "scale": [g["scale"] for g in gs],
        "zero": [g["zero"] for g in gs],
        "res": sum((g["res"] for g in gs), []),
        "rscale": [g["rscale"] for g in gs],
        "deq2": sum((g["deq2"] for g in gs), []),
        "khat": sum((g["khat"] for g in gs), []),
    }


def dot_exact(q: Sequence[float], k: Sequence[Fraction]) -> Fraction:
    return sum((Fraction(a) * b for a, b in zip(q, k)), Fraction(0))


def decode_head(q: Sequence[Sequence[float]], K: Sequence[Sequence[float]],
                V: Sequence[Sequence[float]], L: int, delta: float, sm_scale: float,
                sink: int = 64, local: int = 256, select: str = "union") -> Dict[str, object]:
    """Tiny-input FFD decode for the query heads q (lists of floats) of one KV head.

    select: "union" (every token of the kept blocks), "head_block" (kept blocks
    that are forced or reach the head's own threshold) or "head_token" (support
    tokens and tokens whose estimate reaches the head's threshold)."""
    toks = [pack_token(K[t]) for t in range(L)]
    G = len(q)
    scale = Fraction(sm_scale)
    est = [[float(dot_exact(q[h], toks[t]["deq2"]) * scale) for t in range(L)] for h in range(G)]
    exact = [[float(dot_exact(q[h], toks[t]["khat"]) * scale) for t in range(L)] for h in range(G)]
    support = [t for t in range(L) if t < sink or t >= L - local]
    m_tilde = [max(exact[h][t] for t in support) for h in range(G)]
    thr = [m - delta for m in m_tilde]
    nblk = (L + 63) // 64
    keep, forced, bmax = [], [], []
    for b in range(nblk):
        ts = list(range(64 * b, min(64 * b + 64, L)))
        f = any((t < sink or t >= L - local) for t in ts)
        bm = [max(est[h][t] for t in ts) for h in range(G)]
        forced.append(f)
        bmax.append(bm)
        keep.append(f or any(bm[h] >= thr[h] for h in range(G)))
    out, attended = [], []
    for h in range(G):
        ts = []
        for t in range(L):
            b = t // 64
            if not keep[b]:
                continue
            if select == "head_block" and not (forced[b] or bmax[b][h] >= thr[h]):
                continue
            if select == "head_token" and not (t < sink or t >= L - local or est[h][t] >= thr[h]):
                continue
            ts.append(t)
        attended.append(ts)
        M = max(exact[h][t] for t in ts)
        w = [math.exp(exact[h][t] - M) for t in ts]
        den = math.fsum(w)
        out.append([math.fsum(wi * float(V[t][c]) for wi, t in zip(w, ts)) / den for c in range(len(V[0]))])
    return {"toks": toks, "est": est, "exact": exact, "m_tilde": m_tilde, "thr": thr,
            "bmax": bmax, "forced": forced, "keep": keep, "attended": attended, "out": out}
