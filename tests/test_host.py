"""Host-side behaviour that needs no GPU: the benchmark refuses more than one
GPU, the binding fails loudly when the HIP library is missing (no fallback),
and the carried-state buffer helper has the packed layout's shape."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    from complex_valued_attention_amd import cattn
    monkeypatch.setattr(cattn, "_lib", None)
    monkeypatch.setattr(cattn, "LIB_PATH", str(tmp_path / "missing" / "libcattn.so"))
    with pytest.raises(RuntimeError, match="not built"):
        cattn.lib()


def test_state_buffer_shape():
    torch = pytest.importorskip("torch")
    from complex_valued_attention_amd import cattn
    S = cattn.born_state_buffer(2, 3, 5, device="cpu")
    assert S.dtype == torch.float32 and tuple(S.shape) == (2, 3, 11, 5, 5) and not S.any()


def test_measured_traffic_entries_match_their_sources():
    # a measured-traffic entry is reported only while its kernel source is the
    # one the counters were taken on; every entry in the table must be current
    import hashlib
    import bench
    for name, m in bench.MEASURED_TRAFFIC.items():
        with open(os.path.join(bench.ROOT, m["source"]), "rb") as f:
            assert hashlib.sha256(f.read()).hexdigest() == m["sha256"], name
