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
