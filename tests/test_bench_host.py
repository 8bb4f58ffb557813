"""Host logic of bench.py (no GPU): the one-GPU guard and the lookup of
measured HBM traffic, which must be dropped when the summary covers another
workload or other kernel sources."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, **over):
    t = {"workload": "long_8k", "kernel_source_sha256": bench.kernel_source_hash(),
         "bytes_per_launch": {"bwd_dkdv": 3.25e9, "bwd_dq": 2.66e9}}
    t.update(over)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(t))
    return str(p)


def test_traffic_taken_on_these_sources(tmp_path):
    path = _summary(tmp_path)
    assert bench.measured_traffic(path, "bwd_dkdv", "long_8k") == 3.25e9
    assert bench.measured_traffic(path, "bwd_dq", "long_8k") == 2.66e9
    assert bench.measured_traffic(path, "fwd_main", "long_8k") is None


def test_traffic_of_other_sources_or_workload_is_dropped(tmp_path):
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "bwd_dkdv", "long_8k") is None
    assert bench.measured_traffic(_summary(tmp_path), "bwd_dkdv", "train_4k") is None
    stale = _summary(tmp_path, kernel_source_sha256="0" * 64)
    assert bench.measured_traffic(stale, "bwd_dkdv", "long_8k") is None


def test_source_hash_changes_with_any_kernel_file(tmp_path, monkeypatch):
    """One changed byte in any hashed source gives another hash, so a
    traffic summary is dropped once a kernel source changes."""
    import shutil
    csrc = tmp_path / "bwd_rope_apply_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "bwd_rope_apply_amd", "csrc", name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    assert {"mfma.hip", "tile.h", "common.h"} <= set(bench.KERNEL_SOURCES)
    for name in bench.KERNEL_SOURCES:
        f = csrc / name
        orig = f.read_bytes()
        f.write_bytes(orig + b"\n")
        assert bench.kernel_source_hash() != base, name
        f.write_bytes(orig)
    assert bench.kernel_source_hash() == base
