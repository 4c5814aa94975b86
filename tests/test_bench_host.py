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
    # a summary in the committed file's form, taken on this kernel source
    summary = tmp_path / "counters.txt"
    summary.write_text("# HBM traffic\n\nkernels_sha256: %s\nentry_format: r12\n"
                       "hbm_bytes_per_dispatch: 60321349\n" % bench.kernels_sha())
    monkeypatch.setattr(bench, "COUNTERS", str(summary))
    assert bench.read_counters("r12") == 60321349.0
    assert bench.read_counters("u32") is None  # another entry format
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


def test_committed_summary_has_the_fields_bench_reads():
    kv = {}
    for line in open(bench.COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert len(kv["kernels_sha256"]) == 16 and kv["entry_format"] == "r12"
    assert float(kv["hbm_bytes_per_dispatch"]) > 40e6


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
