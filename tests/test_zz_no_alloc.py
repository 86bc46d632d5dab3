"""GPU check of ffd_decode_attn_noalloc (the allocation-free decode step).

Two calls in a row through the C ABI, the second on a smaller input: each
output must equal ffd_decode_attn's on the same inputs bit for bit (same
kernels and work split, only the workspace differs), and match the fp64
oracle under the GPU's block mask (max-abs 2e-3, rel-L2 1e-3).
"""
import numpy as np
import pytest

from oracle import ffd_oracle as orc
from synthetic import WORKLOADS, Workload, make_case
from tests.gpu_helpers import check_head, dev, gpu_decode, gpu_pack, say, shape_for, torch_mod, SM_SCALE

pytestmark = pytest.mark.gpu


def _compare(w, seed, delta, heads, torch, fill_out):
    import sparse_long_context_ffd_amd as ffd
    c = make_case(w, seed, heads=heads)
    shape = shape_for(w)
    qd, ld = dev(c["q"], torch), dev(c["seq_lens"], torch)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    say(f"noalloc {w.name} seed={seed} delta={delta} heads={heads}")
    # the existing entry point, with its diagnostics (mask for the oracle check)
    ref = gpu_decode(shape, qd, cache, ld, delta, torch)
    out = torch.full((w.batch, w.q_heads, 128), fill_out, dtype=torch.float16, device="cuda")
    ffd.decode_attn_noalloc(shape, qd, cache, ld, delta, SM_SCALE, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.array_equal(got, ref["out"]), f"{w.name}: noalloc output differs from ffd_decode_attn"
    G = w.group
    for b, h in heads:
        pk = orc.quantize_k(c["k"][b, h])
        check_head(orc, c["q"][b, h * G:(h + 1) * G], pk, c["v"][b, h], int(c["seq_lens"][b]), delta,
                   {**ref, "out": got}, b, h, G, label=f"noalloc {w.name} b{b} h{h}")
    return got


def test_noalloc_matches_workspace_call_twice_then_smaller():
    torch = torch_mod()
    # first call: the 16K Llama-like layer (every KV head); second: a smaller
    # ragged batch with another group size, on the same static scratch
    big = WORKLOADS["llama8b_16k"]
    _compare(big, 1, 5.0, [(0, h) for h in range(big.kv_heads)], torch, np.nan)
    small = Workload("noalloc_small", 2, 6, 2, 2048, None, len_range=(300, 2048), deltas=(3.0,), needles=4)
    _compare(small, 0, 3.0, [(b, h) for b in range(2) for h in range(2)], torch, np.nan)
    # and the big one again, after the scratch held the small call's contents
    _compare(big, 2, 7.0, [(0, 0), (0, 5)], torch, 0.0)
