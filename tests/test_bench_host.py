"""Host-side parts of bench.py that decide what its JSON line reports (no
GPU): roofline.traffic comes from the committed counter summary only while
that summary matches the kernel source and the entry format being timed, and
a run on more than one GPU is refused before any device work."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counters_gate_on_kernel_source_and_format(tmp_path, monkeypatch):
    assert os.path.exists(bench.COUNTERS)
    # the committed summary matches the committed kernels and the r12 format
    traffic = bench.read_counters("r12")
    assert traffic is not None and traffic > 40e6
    assert bench.read_counters("u32") is None
    # a kernel source that differs by one byte: no traffic
    src = tmp_path / "kernels.hip"
    shutil.copy(bench.KERNEL_SRC, src)
    with open(src, "a") as f:
        f.write("\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    assert bench.read_counters("r12") is None
    # no summary at all: no traffic
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.txt"))
    assert bench.read_counters("r12") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
