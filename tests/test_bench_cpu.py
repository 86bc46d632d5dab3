"""Host-side checks of bench.py's contract (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_traffic_is_null_for_other_sources():
    import bench
    assert bench.traffic_bytes("no_such_workload") is None
    saved = dict(bench.TRAFFIC_KIB)
    try:
        bench.TRAFFIC_KIB["llama8b_16k"] = dict(saved["llama8b_16k"], sources="0" * 16)
        assert bench.traffic_bytes("llama8b_16k") is None
        bench.TRAFFIC_KIB["llama8b_16k"] = dict(saved["llama8b_16k"], sources=bench.kernel_digest())
        t = bench.traffic_bytes("llama8b_16k")
        rec = saved["llama8b_16k"]
        assert t == int(round((rec["fetch"] * bench.FETCH_SCALE + rec["write"] * bench.WRITE_SCALE) * 1024))
    finally:
        bench.TRAFFIC_KIB.clear()
        bench.TRAFFIC_KIB.update(saved)


def test_digest_ignores_comments_not_code(tmp_path, monkeypatch):
    import shutil
    import bench
    pkg = tmp_path / "sparse_long_context_ffd_amd"
    shutil.copytree(os.path.join(ROOT, "sparse_long_context_ffd_amd", "csrc"), pkg / "csrc")
    shutil.copy(os.path.join(ROOT, "sparse_long_context_ffd_amd", "build.py"), pkg / "build.py")
    (tmp_path / "include").mkdir()
    shutil.copy(os.path.join(ROOT, "include", "ffd.h"), tmp_path / "include" / "ffd.h")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_digest()
    assert d0 == json.loads(json.dumps(d0)) and len(d0) == 16
    src = pkg / "csrc" / "ffd_decode.hip"
    text = src.read_text()
    src.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3))
    assert bench.kernel_digest() == d0  # comments and whitespace do not count
    src.write_text(text.replace("kWaves", "kWavez"))
    assert bench.kernel_digest() != d0  # code does


def test_rotation_reads_more_than_a_gigabyte_between_visits():
    """R copies: R - 1 steps of reads between two visits of one copy exceed
    TOUCH_BETWEEN_VISITS (> 1 GB, four times the 256 MB MALL)."""
    import bench
    assert bench.TOUCH_BETWEEN_VISITS > 1e9
    for read, stored in [(20.5e6, 57.7e6), (273e6, 923e6), (1.07e9, 1.07e9), (6.3e6, 57.7e6), (2e9, 2e9)]:
        R = bench.copies_for(read, stored)
        assert R >= 2
        assert (R - 1) * read >= bench.TOUCH_BETWEEN_VISITS
        assert R * stored <= max(bench.ROTATE_BUDGET, 2 * stored)
    # the memory budget caps the copies (and then says so in the log, not silently)
    assert bench.copies_for(1e3, 10e9) == int(bench.ROTATE_BUDGET // 10e9)


def test_sweep_workloads_match_the_16k_and_256k_needle_counts():
    import bench
    from synthetic import WORKLOADS
    for name, L in (("llama8b_16k", 16384), ("long_256k", 262144)):
        w, s = WORKLOADS[name], bench.sweep_workload(L)
        assert (s.batch, s.q_heads, s.kv_heads, s.max_len, s.seq_len, s.needles) == \
               (w.batch, w.q_heads, w.kv_heads, w.max_len, w.seq_len, w.needles)
    assert [bench.sweep_workload(L).needles for L in (32768, 65536, 131072)] == [23, 32, 45]


def test_unknown_leg_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--legs", "long,nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "nope" in r.stderr
