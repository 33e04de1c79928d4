"""Host-side logic of bench.py (CPU): the pair counts behind the reported TFLOP/s, the refusal
of multi-GPU runs, and the guard that drops measured HBM traffic once a kernel's code changes."""
import json
import os
import subprocess
import sys

import pytest

import bench
from oracle import ttt_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("L", [1, 7, 32, 45])
@pytest.mark.parametrize("step", [0, 1, 3])
def test_pair_counts_match_the_mask(L, step):
    """bench's closed forms for |M_causal| and |M| against the oracle's mask, counted."""
    for T in sorted({0, 1, L // 3, L - 1, L}):
        causal = int(O.mask(L, 0, T).sum())
        assert bench.causal_pairs(L, T) == causal
        assert bench.total_pairs(L, step, T) == O.unmasked_pairs(L, step, T)


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    name = "bwd_dkdv_mfma"
    digest = bench.source_digest((bench.kernel_source(name), "common.cuh"))
    rec = {bench.TRAFFIC_TAG[2]: {"kernels": {name: {"bytes_per_launch": 123,
                                                       "code_digest": digest}}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(2, name) == 123
    assert bench.measured_traffic(3, name) is None          # no record for that workload
    assert bench.measured_traffic(2, "fwd_causal_mfma") is None
    rec[bench.TRAFFIC_TAG[2]]["kernels"][name]["code_digest"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic(2, name) is None          # code changed since the counters


def test_traffic_only_for_the_profiled_paths(monkeypatch):
    """The counters were taken on the per-step, stored-dS, fused-suffix launches; other paths
    run the kernels differently, so they get no traffic figure."""
    monkeypatch.setattr(bench, "measured_traffic", lambda config, name: 7)
    assert bench.run_traffic(2, "bwd_dkdv_mfma", False, "stored", "fused") == 7
    assert bench.run_traffic(2, "bwd_dkdv_mfma", True, "stored", "fused") is None
    assert bench.run_traffic(2, "bwd_dkdv_mfma", False, "recompute", "fused") is None
    assert bench.run_traffic(2, "bwd_dkdv_mfma", False, "fused-suffix", "fused") is None
    assert bench.run_traffic(2, "bwd_dkdv_mfma", False, "stored", "dense") is None


def test_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n/* block */\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    a = bench.source_digest(("k.hip",))
    src.write_text("int f() {\n  return 1;  // another comment\n}\n")
    assert bench.source_digest(("k.hip",)) == a
    src.write_text("int f() { return 2; }\n")
    assert bench.source_digest(("k.hip",)) != a
