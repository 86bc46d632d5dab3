"""Plain fp64 oracle of one FFD decode-attention step (test infrastructure only).

Source: "Faster Than Flash: Exploiting Attention Sparsity for Efficient
Long-Context Decoding" (gist.science technical summary of arXiv 2609.00097).
Sections cited below are that page's Method sections:

* M1 "content-aware scanning via low-bit quantization": K is stored as a
  2-bit thumbnail (used to estimate scores) plus 8-bit residuals that
  rebuild K close to fp16 for the final computation.
* M2 "Top-delta selection": token j is kept when s_j >= m~ - delta, where
  m~ is a pseudo-max taken over the sink (initial) tokens and the local
  window only; delta = 5 keeps tokens whose weight exceeds e^-5 of the peak,
  so scores are natural-log softmax logits.
* M3 "fused kernel", three stages: (1) pseudo-max from sink and local
  tokens, (2) stream the 2-bit keys, compute provisional scores and filter
  blocks against the threshold, (3) for the selected blocks load the 8-bit
  residuals and the values and compute exact attention.

Readings where the page leaves a step open (each is listed with its reason
in the design notes of the repository):

* The page does not define the quantizer.  Per token and per 32-channel
  group: zero = group min; scale = fp16(RNE((max - min) / 3)); a signed
  zero in either is stored as +0; 2-bit code
  = number of k in {1,2,3} with x - zero >= (k - 1/2) scale (0 when scale
  is 0); residual r = x - (zero + code * scale); residual scale =
  fp16(RNE(max|r| / 127)); int8 residual = sign(r) * min(127, number of
  k >= 1 with |r| >= (k - 1/2) rscale) (0 when rscale is 0);
  K-hat = zero + code*scale + res*rscale.
* "Exact" scores use K-hat (the cache holds K only as thumbnail +
  residual); estimated scores use the thumbnail zero + code*scale.
* Blocks of 64 tokens.  A block is kept when it contains a sink/local
  token, or when for some query head of the GQA group its largest estimated
  score reaches that head's threshold.  Every query head of the group
  attends to every valid token of every kept block.
* Sink = the first 64 tokens, local = the last 256 tokens.
* Dropped tokens contribute nothing; the softmax is renormalised over the
  kept tokens (stage 3 computes exact attention on the kept blocks).

All fp16 inputs convert to fp64 exactly; with the conventions above every
quantizer decision is an exact fp64 comparison and ``f16_round`` of an fp64
quotient equals round-to-nearest-even of the exact rational (the quotient
is far from every fp16 rounding midpoint relative to fp64 error).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
BLOCK = 64
GROUP = 32
N_GROUPS = HEAD_DIM // GROUP
CODE_MAX = 3
RES_MAX = 127


def f16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest fp16 value (ties to even); return fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# M1: thumbnail + residual representation of K
# --------------------------------------------------------------------------
def quantize_k(K16: np.ndarray) -> Dict[str, np.ndarray]:
    """Quantize fp16 keys ``[..., 128]`` per token and 32-channel group.

    Returns logical (unpacked) fields:
    ``codes`` uint8 [...,128] in 0..3, ``scale``/``zero`` fp16 [...,4],
    ``res`` int8 [...,128] in -127..127, ``rscale`` fp16 [...,4].
    """
    K16 = np.asarray(K16)
    assert K16.dtype == np.float16 and K16.shape[-1] == HEAD_DIM
    lead = K16.shape[:-1]
    x = K16.astype(np.float64).reshape(lead + (N_GROUPS, GROUP))

    zero = x.min(axis=-1) + 0.0          # a signed-zero minimum is stored as +0
    scale = f16_round((x.max(axis=-1) - zero) / 3.0) + 0.0
    d = x - zero[..., None]
    s = scale[..., None]
    # count of thresholds (k - 1/2) * scale, k = 1..3, that x - zero reaches
    codes = sum((d >= (k - 0.5) * s).astype(np.int64) for k in range(1, CODE_MAX + 1))
    codes = np.where(s > 0, codes, 0)

    deq2 = zero[..., None] + codes * s
    r = x - deq2
    rscale = f16_round(np.abs(r).max(axis=-1) / float(RES_MAX))
    a = np.abs(r)
    s8 = rscale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        k = np.floor(np.where(s8 > 0, a / s8, 0.0) + 0.5)
    # make k exactly #{j >= 1 : |r| >= (j - 1/2) * rscale}; both products are exact in fp64
    k = k + (a >= (k + 0.5) * s8)
    k = k - ((k > 0) & (a < (k - 0.5) * s8))
    k = np.minimum(k, RES_MAX)
    res = np.where(s8 > 0, np.sign(r) * k, 0.0)

    return {
        "codes": codes.reshape(lead + (HEAD_DIM,)).astype(np.uint8),
        "scale": scale.astype(np.float16),
        "zero": zero.astype(np.float16),
        "res": res.reshape(lead + (HEAD_DIM,)).astype(np.int8),
        "rscale": rscale.astype(np.float16),
    }


def dequantize(pk: Dict[str, np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """(thumbnail keys zero + code*scale, full keys K-hat) in fp64, shape [..., 128]."""
    c = pk["codes"].astype(np.float64)
    lead = c.shape[:-1]
    c = c.reshape(lead + (N_GROUPS, GROUP))
    e = pk["res"].astype(np.float64).reshape(lead + (N_GROUPS, GROUP))
    s = pk["scale"].astype(np.float64)[..., None]
    z = pk["zero"].astype(np.float64)[..., None]
    s8 = pk["rscale"].astype(np.float64)[..., None]
    deq2 = z + c * s
    khat = deq2 + e * s8
    return deq2.reshape(lead + (HEAD_DIM,)), khat.reshape(lead + (HEAD_DIM,))


def slice_tokens(pk: Dict[str, np.ndarray], lo: int, hi: int) -> Dict[str, np.ndarray]:
    """Token range [lo, hi) of a packed single-head cache (leading axis = token)."""
    return {k: v[lo:hi] for k, v in pk.items()}


# --------------------------------------------------------------------------
# scores, supports and blocks
# --------------------------------------------------------------------------
def scores(q16: np.ndarray, keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax logits s[h, t] = (q_h . key_t) * sm_scale in fp64; q16 [G][128], keys [L][128]."""
    q = np.asarray(q16).astype(np.float64)
    return (q @ np.asarray(keys, dtype=np.float64).T) * float(sm_scale)


def support_mask(L: int, sink: int, local: int) -> np.ndarray:
    """Tokens the pseudo-max looks at: [0, min(sink, L)) U [max(0, L - local), L)."""
    m = np.zeros(L, dtype=bool)
    m[: min(sink, L)] = True
    m[max(0, L - local): L] = True
    return m


def n_blocks(L: int) -> int:
    return (L + BLOCK - 1) // BLOCK


def forced_blocks(L: int, sink: int, local: int) -> np.ndarray:
    """Blocks holding at least one sink or local token (always kept)."""
    sup = support_mask(L, sink, local)
    nb = n_blocks(L)
    pad = np.zeros(nb * BLOCK, dtype=bool)
    pad[:L] = sup
    return pad.reshape(nb, BLOCK).any(axis=1)


def block_max(s: np.ndarray, L: int) -> np.ndarray:
    """Per-head maximum of s[:, t] over the valid tokens of each 64-token block."""
    G = s.shape[0]
    nb = n_blocks(L)
    pad = np.full((G, nb * BLOCK), -np.inf)
    pad[:, :L] = s[:, :L]
    return pad.reshape(G, nb, BLOCK).max(axis=2)


# --------------------------------------------------------------------------
# exact attention on a token subset, partials and their LSE merge
# --------------------------------------------------------------------------
def attend_tokens(s: np.ndarray, V16: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """softmax(s[:, tokens]) @ V[tokens] in fp64, with the true max over the subset."""
    st = s[:, tokens]
    M = st.max(axis=1, keepdims=True)
    w = np.exp(st - M)
    V = np.asarray(V16, dtype=np.float64)[tokens]
    return (w @ V) / w.sum(axis=1, keepdims=True)


def partial(s: np.ndarray, V16: np.ndarray, tokens: np.ndarray):
    """Un-normalised split partial (o, m, l): o = sum e^{s-m} V, l = sum e^{s-m}, m = max s."""
    if tokens.size == 0:
        G = s.shape[0]
        return np.zeros((G, HEAD_DIM)), np.full(G, -np.inf), np.zeros(G)
    st = s[:, tokens]
    m = st.max(axis=1)
    w = np.exp(st - m[:, None])
    return w @ np.asarray(V16, dtype=np.float64)[tokens], m, w.sum(axis=1)


def lse_merge(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Merge split partials: M = max m_i, out = sum o_i e^{m_i-M} / sum l_i e^{m_i-M}."""
    ms = np.stack([p[1] for p in parts])              # [n][G]
    M = ms.max(axis=0)
    f = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    num = sum(p[0] * f[i][:, None] for i, p in enumerate(parts))
    den = sum(p[2] * f[i] for i, p in enumerate(parts))
    return num / den[:, None]


# --------------------------------------------------------------------------
# one decode step for one (sequence, KV head): M3 stages 1-3
# --------------------------------------------------------------------------
SELECTIONS = ("union", "head_block", "head_token")


def decode_head(q16: np.ndarray, pk: Dict[str, np.ndarray], V16: np.ndarray, L: int,
                delta: float, sm_scale: float, sink: int = 64, local: int = 256,
                keep: Optional[np.ndarray] = None, select: str = "union",
                tmask: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """FFD decode attention for the G query heads of one KV head.

    ``pk`` is the packed cache of that KV head (token axis first, at least L
    tokens), ``V16`` fp16 [>=L][128].  ``keep`` overrides the block selection
    and ``tmask`` ([G][L] bool) the tokens each head attends (both used to
    compare outputs under another implementation's decisions).

    ``select`` chooses what each query head attends inside the blocks kept for
    the KV head (the loads stay the kept blocks in every case):

    * "union" -- every valid token of every kept block (the block filter of
      M3 stage 2 shared by the GQA group);
    * "head_block" -- the kept blocks that are forced or whose largest
      estimated score reaches this head's own threshold;
    * "head_token" -- M2's criterion per token and head: the sink and local
      tokens plus every token whose estimated score reaches this head's
      threshold.  (The estimate decides, as it does for blocks: exact scores
      exist only for loaded blocks.)

    Returns m_tilde [G], thr [G], s_est [G][L], s_exact [G][L], bmax [G][nblk],
    forced [nblk], keep [nblk], tmask [G][L], out [G][128] (fp64).
    """
    if select not in SELECTIONS:
        raise ValueError(f"unknown selection {select!r}")
    if L < 1:
        raise ValueError("sequence length must be >= 1")
    deq2, khat = dequantize(slice_tokens(pk, 0, L))
    s_exact = scores(q16, khat, sm_scale)

    # stage 1: pseudo-max over sink and local tokens, per query head
    sup = support_mask(L, sink, local)
    m_tilde = s_exact[:, sup].max(axis=1)
    thr = m_tilde - float(delta)

    # stage 2: provisional scores from the 2-bit thumbnail, block filter
    s_est = scores(q16, deq2, sm_scale)
    bmax = block_max(s_est, L)
    forced = forced_blocks(L, sink, local)
    sel = forced | (bmax >= thr[:, None]).any(axis=0)
    if keep is None:
        keep = sel
    keep = np.asarray(keep, dtype=bool)

    # which tokens each head attends, inside the kept blocks
    G = q16.shape[0]
    tok = np.repeat(keep, BLOCK)[:L]
    if tmask is None:
        if select == "union":
            per_head = np.ones((G, L), dtype=bool)
        elif select == "head_block":
            hb = forced[None, :] | (bmax >= thr[:, None])
            per_head = np.repeat(hb, BLOCK, axis=1)[:, :L]
        else:
            per_head = sup[None, :] | (s_est >= thr[:, None])
        tmask = per_head & tok[None, :]
    tmask = np.asarray(tmask, dtype=bool)
    if tmask.shape != (G, L):
        raise ValueError("tmask must be [G][L]")

    # stage 3: exact attention over each head's attended tokens
    out = np.stack([attend_tokens(s_exact[h:h + 1], V16[:L], np.nonzero(tmask[h])[0])[0] for h in range(G)])
    return {"m_tilde": m_tilde, "thr": thr, "s_est": s_est, "s_exact": s_exact,
            "bmax": bmax, "forced": forced, "keep": keep, "selected": sel, "tmask": tmask, "out": out}


# --------------------------------------------------------------------------
# run-time termination of the refine stream (the ART page, "Attention
# Run-time Termination", Method sections 2.1-2.4)
# --------------------------------------------------------------------------
ART_PROBE = 8  # probe = the first 8 output channels of the group's first query head


def art_streams(nblk: int, stream_blocks: int) -> List[List[int]]:
    """The streams of one sequence: a streaming (split-KV) attention unit
    accumulates a contiguous run of KV blocks, so stream s holds blocks
    [s * stream_blocks, (s + 1) * stream_blocks), cut at the sequence end.
    The partition depends only on the sequence length and the call's
    stream_blocks."""
    if stream_blocks < 1:
        raise ValueError("stream_blocks must be >= 1")
    return [list(range(s, min(s + stream_blocks, nblk))) for s in range(0, nblk, stream_blocks)]


def art_decode_head(q16: np.ndarray, pk: Dict[str, np.ndarray], V16: np.ndarray, L: int,
                    delta: float, sm_scale: float, stream_blocks: int, tau: float, phi: float,
                    patience: int, sink: int = 64, local: int = 256,
                    keep: Optional[np.ndarray] = None) -> Dict[str, object]:
    """FFD decode where every stream of kept blocks may stop early.

    Each stream (``art_streams``) visits its kept blocks in increasing order,
    folding each into a running output.  After block t it takes the probe
    x_t = the first ART_PROBE channels of its running normalised output for
    the group's first query head, and from the second block on compares it
    with the previous probe:
        d_scale = | ||x_t|| - ||x_{t-1}|| |,   d_dir = 1 - cos(x_t, x_{t-1})
    (d_dir = 1 when either norm is 0).  A step is stable when d_scale < tau
    and d_dir < phi; after `patience` consecutive stable steps the stream
    skips its remaining blocks.  Every query head of the group follows the
    stream's decision.  The output is exact attention over the union of the
    visited blocks (the streams' outputs merge by log-sum-exp, which is order
    invariant).  Block 0 (forced kept) is the first block of stream 0, so it
    is always evaluated.  patience <= 0 disables the stop.

    Returns the decode_head fields plus ``visited`` [nblk] bool, ``streams``
    (per stream: blocks, blocks kept, blocks visited, per step (d_scale, d_dir)).
    """
    base = decode_head(q16, pk, V16, L, delta, sm_scale, sink, local, keep=keep)
    keep = base["keep"]
    s = base["s_exact"]
    G = q16.shape[0]
    nblk = n_blocks(L)
    Vf = np.asarray(V16, dtype=np.float64)[:L]
    visited = np.zeros(nblk, dtype=bool)
    streams = []
    for blocks in art_streams(nblk, stream_blocks):
        kept = [b for b in blocks if keep[b]]
        m = np.full(G, -np.inf)
        lsum = np.zeros(G)
        o = np.zeros((G, HEAD_DIM))
        prev = None
        stable = 0
        steps = []
        seen = []
        for b in kept:
            t = np.arange(b * BLOCK, min(b * BLOCK + BLOCK, L))
            mb = s[:, t].max(axis=1)
            mn = np.maximum(m, mb)
            scale = np.where(np.isfinite(m), np.exp(m - mn), 0.0)
            w = np.exp(s[:, t] - mn[:, None])
            o = o * scale[:, None] + w @ Vf[t]
            lsum = lsum * scale + w.sum(axis=1)
            m = mn
            seen.append(b)
            x = o[0, :ART_PROBE] / lsum[0]
            if prev is not None:
                n1, n0 = float(np.linalg.norm(x)), float(np.linalg.norm(prev))
                d_scale = abs(n1 - n0)
                d_dir = 1.0 - float(x @ prev) / (n1 * n0) if n1 > 0.0 and n0 > 0.0 else 1.0
                steps.append((d_scale, d_dir))
                stable = stable + 1 if (d_scale < tau and d_dir < phi) else 0
                if patience > 0 and stable >= patience:
                    break
            prev = x
        visited[seen] = True
        streams.append({"blocks": blocks, "kept": kept, "visited": seen, "steps": steps})
    tok = np.repeat(visited, BLOCK)[:L]
    out = attend_tokens(s, V16[:L], np.nonzero(tok)[0])
    return {**base, "visited": visited, "streams": streams, "out": out}


def art_decode(q: np.ndarray, pk: Dict[str, np.ndarray], v: np.ndarray, seq_lens: Sequence[int],
               delta: float, sm_scale: float, stream_blocks: int, tau: float, phi: float, patience: int,
               sink: int = 64, local: int = 256,
               heads: Optional[Iterable[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], Dict[str, object]]:
    """art_decode_head for every (b, kv_head) (or the listed ones) of a batch;
    shapes as in ``decode``."""
    B, Hq, _ = q.shape
    Hkv = v.shape[1]
    G = Hq // Hkv
    todo = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    return {(b, h): art_decode_head(q[b, h * G:(h + 1) * G], {f: a[b, h] for f, a in pk.items()}, v[b, h],
                                    int(seq_lens[b]), delta, sm_scale, stream_blocks, tau, phi, patience,
                                    sink, local)
            for b, h in todo}


def dense_head(q16: np.ndarray, keys: np.ndarray, V16: np.ndarray, L: int,
               sm_scale: float) -> np.ndarray:
    """Dense decode attention softmax(q k^T * scale) V over tokens [0, L) in fp64."""
    s = scores(q16, np.asarray(keys)[:L], sm_scale)
    return attend_tokens(s, V16[:L], np.arange(L))


# --------------------------------------------------------------------------
# whole-batch wrappers
# --------------------------------------------------------------------------
def quantize_cache(k: np.ndarray) -> Dict[str, np.ndarray]:
    """quantize_k over a [B][Hkv][L_cap][128] fp16 cache."""
    return quantize_k(k)


def decode(q: np.ndarray, pk: Dict[str, np.ndarray], v: np.ndarray, seq_lens: Sequence[int],
           delta: float, sm_scale: float, sink: int = 64, local: int = 256,
           heads: Optional[Iterable[Tuple[int, int]]] = None,
           keep: Optional[np.ndarray] = None,
           select: str = "union") -> Dict[Tuple[int, int], Dict[str, np.ndarray]]:
    """decode_head for every (b, kv_head) (or the listed ones).

    q fp16 [B][Hq][128]; pk fields [B][Hkv][L_cap][...]; v fp16 [B][Hkv][L_cap][128].
    Query head h belongs to KV head h // G.  ``keep`` (optional, [B][Hkv][nblk_cap])
    overrides the selection per head.
    """
    B, Hq, _ = q.shape
    Hkv = v.shape[1]
    G = Hq // Hkv
    todo = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    res = {}
    for b, h in todo:
        L = int(seq_lens[b])
        pkh = {f: a[b, h] for f, a in pk.items()}
        kp = None if keep is None else np.asarray(keep[b, h][: n_blocks(L)], dtype=bool)
        res[(b, h)] = decode_head(q[b, h * G:(h + 1) * G], pkh, v[b, h], L, delta, sm_scale,
                                  sink, local, keep=kp, select=select)
    return res


def dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens: Sequence[int], sm_scale: float,
          heads: Optional[Iterable[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """dense_head for every (b, kv_head) over fp16 keys k [B][Hkv][L_cap][128]."""
    B, Hq, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    todo = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    return {(b, h): dense_head(q[b, h * G:(h + 1) * G], k[b, h], v[b, h], int(seq_lens[b]), sm_scale)
            for b, h in todo}
