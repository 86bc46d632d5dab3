"""Seeded synthetic KV caches shaped like long-context decode workloads.

Recipe (one decode step, one layer):

* Per (batch b, KV head k) an independent generator
  ``np.random.default_rng([seed, b, k])`` draws, in this order:
  K rows ~ N(0, I_128) for all ``L_cap`` positions; 4 distinct outlier
  channels whose K values are multiplied by 5; V rows ~ N(0, I_128);
  the G query vectors of the group ~ N(0, I_128) times ``q_scale``;
  the needle positions.
* Planted keys (unless ``plant`` is False): tokens 0..3 (attention sinks),
  then ``needles`` distinct positions drawn uniformly from
  ``[sink, L - local)`` so they fall outside the sink and local windows.
  Planted key number i (sinks first) targets query head ``i mod G`` of the
  group: the key keeps its norm and is turned to cosine 0.8 with that
  head's fp16-rounded query direction (0.8 along q-hat, 0.6 along the unit
  part of the old key orthogonal to q-hat).
* q, K and V are rounded to fp16 (round to nearest even) at the end.
* Variable lengths draw from ``np.random.default_rng([seed, 0x4C454E])``.

Nothing here computes scores, quantizes or attends.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
N_SINK_KEYS = 4
OUTLIER_CHANNELS = 4
OUTLIER_GAIN = 5.0
PLANT_COS = 0.8
LEN_STREAM = 0x4C454E  # second seed word of the sequence-length generator


@dataclass(frozen=True)
class Workload:
    """One decode-step workload: shapes, selection threshold(s), generator knobs."""

    name: str
    batch: int
    q_heads: int
    kv_heads: int
    max_len: int                     # L_cap, a multiple of 64
    seq_len: Optional[int]           # fixed length, or None for a uniform draw
    len_range: Optional[Tuple[int, int]] = None  # inclusive range when seq_len is None
    deltas: Tuple[float, ...] = (5.0,)
    needles: int = 0
    plant: bool = True
    q_scale: float = 1.0
    sink: int = 64
    local: int = 256
    note: str = ""

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny_h4x1_4k", 1, 4, 1, 4096, 4096, deltas=(5.0,), needles=8,
                 note="B=1, Hq=4, Hkv=1, L=4096; small enough for the oracle in seconds"),
        Workload("llama8b_16k", 1, 32, 8, 16384, 16384, deltas=(5.0, 7.0), needles=16,
                 note="Llama-3.1-8B-like decode layer at 16K context"),
        Workload("long_256k", 1, 32, 8, 262144, 262144, deltas=(5.0,), needles=64,
                 note="Llama-8B-like heads at 256K context (about 1 GB of fp16 K+V)"),
        Workload("qwen7b_b16_16k32k", 16, 28, 4, 32768, None, len_range=(16384, 32768),
                 deltas=(7.0,), needles=16,
                 note="Qwen2.5-7B-like heads, batch 16, lengths uniform in [16K, 32K]"),
        Workload("stress_b4_128k", 4, 32, 8, 131072, 131072, deltas=(7.0,), needles=0,
                 plant=False, q_scale=0.1,
                 note="low-sparsity stress: q scaled by 0.1, nothing planted"),
    )
}


def seq_lens_for(w: Workload, seed: int) -> np.ndarray:
    """Per-sequence lengths (int32[B]) of workload ``w`` for ``seed``."""
    if w.seq_len is not None:
        return np.full(w.batch, w.seq_len, dtype=np.int32)
    lo, hi = w.len_range
    rng = np.random.default_rng([seed, LEN_STREAM])
    return rng.integers(lo, hi, size=w.batch, endpoint=True).astype(np.int32)


def planted_positions(w: Workload, L: int, rng: np.random.Generator) -> np.ndarray:
    """Sink positions 0..3 followed by distinct needle positions in [sink, L-local)."""
    lo, hi = w.sink, L - w.local
    n = min(w.needles, max(hi - lo, 0))
    needles = (rng.choice(hi - lo, size=n, replace=False) + lo) if n > 0 else np.zeros(0, np.int64)
    sinks = np.arange(min(N_SINK_KEYS, L))
    return np.concatenate([sinks, needles.astype(np.int64)])


def _plant(K: np.ndarray, pos: np.ndarray, q16: np.ndarray) -> None:
    G = q16.shape[0]
    qd = q16.astype(np.float64)
    qhat = qd / np.linalg.norm(qd, axis=1, keepdims=True)
    for i, t in enumerate(pos):
        u = qhat[i % G]
        k = K[t]
        nk = np.linalg.norm(k)
        w = k - np.dot(k, u) * u
        nw = np.linalg.norm(w)
        if nw == 0.0:
            # degenerate: key parallel to q; pick any unit vector orthogonal to u
            e = np.zeros_like(u)
            e[int(np.argmin(np.abs(u)))] = 1.0
            w = e - np.dot(e, u) * u
            nw = np.linalg.norm(w)
        K[t] = nk * (PLANT_COS * u + np.sqrt(1.0 - PLANT_COS ** 2) * (w / nw))


def make_head(w: Workload, seed: int, b: int, kvh: int, L: int):
    """Generate one (batch, KV head) slice.

    Returns ``(q16 [G][128], K16 [L_cap][128], V16 [L_cap][128])`` as float16.
    Rows at positions >= L are valid random data that a correct kernel never
    attends to.  The slice depends only on (seed, b, kvh, L).
    """
    n = w.max_len
    rng = np.random.default_rng([seed, b, kvh])
    K = rng.standard_normal((n, HEAD_DIM))
    ch = rng.choice(HEAD_DIM, size=OUTLIER_CHANNELS, replace=False)
    K[:, ch] *= OUTLIER_GAIN
    V = rng.standard_normal((n, HEAD_DIM))
    q = rng.standard_normal((w.group, HEAD_DIM)) * w.q_scale
    q16 = q.astype(np.float16)
    if w.plant:
        _plant(K, planted_positions(w, L, rng), q16)
    return q16, K.astype(np.float16), V.astype(np.float16)


def make_case(w: Workload, seed: int, heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Generate the whole workload (or a subset of (b, kv_head) slices).

    Returns a dict with ``q`` fp16 [B][Hq][128], ``k`` and ``v`` fp16
    [B][Hkv][L_cap][128], ``seq_lens`` int32 [B].  Slices not listed in
    ``heads`` are left zero.
    """
    lens = seq_lens_for(w, seed)
    G = w.group
    q = np.zeros((w.batch, w.q_heads, HEAD_DIM), np.float16)
    k = np.zeros((w.batch, w.kv_heads, w.max_len, HEAD_DIM), np.float16)
    v = np.zeros_like(k)
    todo = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)] if heads is None else list(heads)
    for b, h in todo:
        q16, K16, V16 = make_head(w, seed, b, h, int(lens[b]))
        q[b, h * G:(h + 1) * G] = q16
        k[b, h] = K16
        v[b, h] = V16
    return {"q": q, "k": k, "v": v, "seq_lens": lens}
