"""Host-side checks of bench.py (no GPU): the causal pair counts behind every algorithmic flop
figure, the flop count of the training shape, the one-GPU guard, and that a stored HBM traffic
figure is reported only for the sources it was measured on."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(lengths, cb):
    """Every causal pair (i, j <= i) of every sequence, classified by the distance of their chunks."""
    out = {"all": 0, "same": 0, "adj": 0, "far": 0}
    for L in lengths:
        for i in range(L):
            for j in range(i + 1):
                d = i // cb - j // cb
                out["all"] += 1
                out["same" if d == 0 else "adj" if d == 1 else "far"] += 1
    return out


@pytest.mark.parametrize("lengths,cb", [([1], 4), ([7, 4, 1], 4), ([9, 16, 17, 33], 4), ([300, 129, 1], 128)])
def test_pair_counts_match_brute_force(lengths, cb):
    got = bench.pair_counts(lengths, cb=cb)
    ref = brute_pairs(lengths, cb)
    assert got["all"] == ref["all"]
    assert got["same"] == ref["same"]
    assert got["adj"] == ref["adj"]
    assert got["far"] == ref["far"]
    assert got["inter"] == ref["adj"] + ref["far"]


def test_training_shape_flops():
    """B=4, T=8192, Hq=16, dk=dv=128: 2 (dk + dv) flop per causal pair and head forward,
    2 (3 dk + 2 dv) backward."""
    pairs = bench.pair_counts([8192] * 4)["all"]
    assert pairs == 4 * 8192 * 8193 // 2
    fwd = 2 * (128 + 128) * pairs * 16
    bwd = 2 * (3 * 128 + 2 * 128) * pairs * 16
    assert fwd == 1099645845504
    assert fwd + bwd == 3848760459264


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    good = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC", {"k": {"bytes": 123, "sha": good, "files": ["kernel.hip"]}})
    assert bench.measured_traffic("k") == 123
    assert bench.measured_traffic("other") is None
    src.write_text("// a kernel, changed\n")
    assert bench.measured_traffic("k") is None

