"""GPU parity of the K-cache pack (ffd_quantize_k): bit-exact with the oracle."""
import numpy as np
import pytest

from oracle import ffd_oracle as orc
from synthetic import WORKLOADS, make_case, make_head
from tests.gpu_helpers import cache_to_host, dev, gpu_pack, say, shape_for, torch_mod
from tests.layout import decode_cache

pytestmark = pytest.mark.gpu
FIELDS = ("codes", "scale", "zero", "res", "rscale")


def _assert_fields_equal(got, ref, label):
    for f in FIELDS:
        a, r = got[f], ref[f]
        if a.dtype == np.float16:
            a, r = a.view(np.uint16), r.view(np.uint16)
        bad = np.argwhere(a != r)
        assert bad.size == 0, f"{label}: field {f} differs at {bad[:5].tolist()} (got {a[tuple(bad[0])]}, ref {r[tuple(bad[0])]})"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_tiny_bit_exact(seed):
    torch = torch_mod()
    w = WORKLOADS["tiny_h4x1_4k"]
    say(f"pack tiny seed={seed}")
    c = make_case(w, seed)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch))
    got = decode_cache(**cache_to_host(cache), B=w.batch, Hkv=w.kv_heads, L_cap=w.max_len)
    ref = orc.quantize_k(c["k"])
    _assert_fields_equal(got, ref, f"tiny seed {seed}")


@pytest.mark.parametrize("name,heads", [("llama8b_16k", [(0, 0), (0, 5)]), ("qwen7b_b16_16k32k", [(3, 2), (15, 0)])])
def test_pack_sampled_heads_bit_exact(name, heads):
    torch = torch_mod()
    w = WORKLOADS[name]
    say(f"pack {name} heads={heads}")
    c = make_case(w, 0, heads=heads)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch))
    got = decode_cache(**cache_to_host(cache), B=w.batch, Hkv=w.kv_heads, L_cap=w.max_len)
    for b, h in heads:
        ref = orc.quantize_k(c["k"][b, h])
        _assert_fields_equal({f: got[f][b, h] for f in FIELDS}, ref, f"{name} b{b} h{h}")


def _edge_keys(rng):
    rows = [rng.standard_normal(128), np.full(128, 0.75), np.zeros(128), rng.standard_normal(128) * 2.0 ** -20,
            rng.standard_normal(128) * 2.0 ** 12, -0.0 * np.ones(128)]
    c = rng.integers(0, 4, 128); c[0] = 0; c[1] = 3
    rows.append(-1.5 + c * 0.25)
    x = np.zeros(128); x[1] = 3.0; x[2:6] = [0.5, 1.5, 2.5, 1.0]; rows.append(x)
    x = rng.standard_normal(128) * 2.0 ** rng.integers(-14, 8, 128); rows.append(x)
    x = np.zeros(128); x[1] = 3 * 2.0 ** -14; x[2] = 2.0 ** -14 + 2.0 ** -24; rows.append(x)
    x = rng.standard_normal(128); x[[3, 40, 77, 120]] *= 5; rows.append(x)
    rows.append(np.full(128, 65504.0)); rows.append(np.linspace(-65504, 65504, 128))
    return np.stack(rows)


def test_pack_edge_values_bit_exact():
    torch = torch_mod()
    rng = np.random.default_rng(11)
    L_cap = 256
    k = rng.standard_normal((2, 3, L_cap, 128))
    edges = _edge_keys(rng)
    k[0, 1, 5:5 + len(edges)] = edges
    k[1, 2, 130:130 + len(edges)] = edges[::-1]
    k = k.astype(np.float16)
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(2, 6, 3, L_cap)
    say("pack edge values")
    cache = gpu_pack(shape, dev(k, torch))
    got = decode_cache(**cache_to_host(cache), B=2, Hkv=3, L_cap=L_cap)
    _assert_fields_equal(got, orc.quantize_k(k), "edge values")


def test_pack_token_range_leaves_other_bytes_untouched():
    """Packing [t_begin, t_end) writes exactly those tokens (1-token append included)."""
    torch = torch_mod()
    rng = np.random.default_rng(3)
    L_cap = 512
    k = rng.standard_normal((1, 2, L_cap, 128)).astype(np.float16)
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(1, 2, 2, L_cap)
    kd = dev(k, torch)
    full = decode_cache(**cache_to_host(gpu_pack(shape, kd)), B=1, Hkv=2, L_cap=L_cap)
    for (t0, t1) in [(100, 101), (63, 200), (0, 1), (511, 512), (130, 130)]:
        say(f"pack range [{t0},{t1})")
        cache = gpu_pack(shape, kd, fill=0xAB, t_begin=t0, t_end=t1)
        raw = cache_to_host(cache)
        got = decode_cache(**raw, B=1, Hkv=2, L_cap=L_cap)
        sel = np.zeros(L_cap, bool)
        sel[t0:t1] = True
        for f in FIELDS:
            a, r = got[f], full[f]
            if a.dtype == np.float16:
                a, r = a.view(np.uint16), r.view(np.uint16)
            assert (a[:, :, sel] == r[:, :, sel]).all(), f"range [{t0},{t1}) field {f}"
        # bytes of untouched tokens keep the fill value
        filled = cache_to_host(gpu_pack(shape, kd, fill=0xAB, t_begin=0, t_end=0))
        unt = decode_cache(**filled, B=1, Hkv=2, L_cap=L_cap)
        for f in FIELDS:
            a, u = got[f], unt[f]
            if a.dtype == np.float16:
                a, u = a.view(np.uint16), u.view(np.uint16)
            assert (a[:, :, ~sel] == u[:, :, ~sel]).all(), f"range [{t0},{t1}) touched other tokens in {f}"


@pytest.mark.parametrize("name,heads", [("tiny_h4x1_4k", None), ("qwen7b_b16_16k32k", [(3, 2), (15, 0)])])
def test_pack_v_tiled_bit_exact(name, heads):
    """ffd_pack_v moves every fp16 value unchanged into the token-quad tiled layout."""
    torch = torch_mod()
    w = WORKLOADS[name]
    say(f"pack_v {name} heads={heads}")
    c = make_case(w, 0, heads=heads)
    shape = shape_for(w)
    cache = gpu_pack(shape, dev(c["k"], torch), dev(c["v"], torch))
    got = decode_cache(**cache_to_host(cache), B=w.batch, Hkv=w.kv_heads, L_cap=w.max_len)["v"]
    for b, h in heads or [(0, 0)]:
        assert np.array_equal(got[b, h].view(np.uint16), c["v"][b, h].view(np.uint16)), f"{name} b{b} h{h}"


def test_pack_v_token_range_leaves_other_bytes_untouched():
    """Ranges that start or end inside a 4-token quad write exactly their tokens."""
    torch = torch_mod()
    rng = np.random.default_rng(5)
    L_cap = 512
    v = rng.standard_normal((2, 2, L_cap, 128)).astype(np.float16)
    k = np.zeros_like(v)
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(2, 4, 2, L_cap)
    kd, vd = dev(k, torch), dev(v, torch)
    for (t0, t1) in [(100, 101), (63, 200), (0, 1), (511, 512), (130, 130), (2, 7), (5, 6), (0, 512)]:
        say(f"pack_v range [{t0},{t1})")
        cache = ffd.PackedCache(shape).fill_(0xAB)
        ffd.pack_v(shape, vd, t0, t1, cache)
        got = decode_cache(**cache_to_host(cache), B=2, Hkv=2, L_cap=L_cap)["v"].view(np.uint16)
        sel = np.zeros(L_cap, bool)
        sel[t0:t1] = True
        assert (got[:, :, sel] == v.view(np.uint16)[:, :, sel]).all(), f"range [{t0},{t1})"
        assert (got[:, :, ~sel] == 0xABAB).all(), f"range [{t0},{t1}) touched other tokens"


def test_append_kv_matches_oracle_and_skips_out_of_range():
    """ffd_append_kv writes, for each sequence, exactly the token at its device
    position: key bytes equal the oracle's quantization of the new key, the
    value lands unchanged in the tiled layout, positions outside [0, L_cap)
    write nothing, and every other byte keeps its fill."""
    torch = torch_mod()
    rng = np.random.default_rng(21)
    B, Hkv, L_cap = 6, 2, 256
    k = rng.standard_normal((B, Hkv, 128))
    k[1, 0, [3, 50, 97]] *= 5
    edges = _edge_keys(rng)
    k[2, 1] = edges[6]                       # on-grid values: zero residual
    k[3, 0] = edges[1]                       # constant group values
    k[5, 1] = edges[12]                      # full fp16 range
    k = k.astype(np.float16)
    v = rng.standard_normal((B, Hkv, 128)).astype(np.float16)
    pos = np.array([0, 65, 130, 255, -1, 256], np.int32)   # quad offsets 0..3, then two skips
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(B, 2 * Hkv, Hkv, L_cap)
    say("append_kv ragged positions")
    cache = ffd.PackedCache(shape).fill_(0xAB)
    ffd.append_kv(shape, dev(k, torch), dev(v, torch), dev(pos, torch), cache)
    torch.cuda.synchronize()
    got = decode_cache(**cache_to_host(cache), B=B, Hkv=Hkv, L_cap=L_cap)
    unt = decode_cache(**cache_to_host(ffd.PackedCache(shape).fill_(0xAB)), B=B, Hkv=Hkv, L_cap=L_cap)
    for b in range(B):
        for h in range(Hkv):
            sel = np.zeros(L_cap, bool)
            if 0 <= pos[b] < L_cap:
                sel[pos[b]] = True
                ref = orc.quantize_k(k[b, h][None])
                ref = {f: ref[f][0] for f in FIELDS}
                ref["v"] = v[b, h]
                _assert_fields_equal({f: got[f][b, h, pos[b]][None] for f in FIELDS},
                                     {f: ref[f][None] for f in FIELDS}, f"append b{b} h{h}")
                assert np.array_equal(got["v"][b, h, pos[b]].view(np.uint16), v[b, h].view(np.uint16)), \
                    f"append value b{b} h{h}"
            for f in FIELDS + ("v",):
                a, u = got[f][b, h], unt[f][b, h]
                if a.dtype == np.float16:
                    a, u = a.view(np.uint16), u.view(np.uint16)
                assert (a[~sel] == u[~sel]).all(), f"append b{b} h{h} touched other tokens in {f}"


def test_append_kv_equals_range_pack():
    """Appending tokens one call at a time gives the same cache bytes as one
    ffd_quantize_k + ffd_pack_v over the whole range."""
    torch = torch_mod()
    rng = np.random.default_rng(22)
    B, Hkv, L_cap = 2, 3, 128
    k = rng.standard_normal((B, Hkv, L_cap, 128)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, L_cap, 128)).astype(np.float16)
    import sparse_long_context_ffd_amd as ffd
    shape = ffd.make_shape(B, Hkv, Hkv, L_cap)
    full = cache_to_host(gpu_pack(shape, dev(k, torch), dev(v, torch), fill=0x5C, t_begin=10, t_end=80))
    cache = ffd.PackedCache(shape).fill_(0x5C)
    pos = torch.tensor([10, 10], dtype=torch.int32, device="cuda")
    say("append_kv 70 steps vs range pack")
    for t in range(10, 80):
        kn = dev(np.ascontiguousarray(k[:, :, t]), torch)
        vn = dev(np.ascontiguousarray(v[:, :, t]), torch)
        ffd.append_kv(shape, kn, vn, pos, cache)
        pos += 1
    torch.cuda.synchronize()
    got = cache_to_host(cache)
    for f in ("codes", "sz", "res", "rscale", "v"):
        assert np.array_equal(got[f], full[f]), f"append loop differs from range pack in {f}"
