"""Build libeffort.so (HIP for gfx950 + host C++) in-tree with hipcc.

    python dynamic_sparsity_approximate_amd/build.py
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libeffort.so")
ARCH = os.environ.get("EFFORT_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# fp contraction off: the keep test multiplies |v_i| by |w| exactly once with
# round-to-nearest; denormals kept (fp16 subnormal weights are exact in fp32);
# float atomics compile to hardware ds_add_f32 / global_atomic_add_f32;
# packed fp32 instructions disabled.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-ffp-contract=off"]
# The atomic optimizer is off so that a returning atomic is waited for where
# its value is used, not at once: the optimizer makes it one atomic per wave
# followed at once by per-lane offsets, and the dispatch issues its
# candidate-slot reservation early precisely to use the result last.
DEVICE = ["--offload-arch=" + ARCH, "-munsafe-fp-atomics", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]

SOURCES = [
    ("kernels.hip", DEVICE + ["-x", "hip"]),
    ("api.cpp", ["-D__HIP_PLATFORM_AMD__"]),
    ("convert.cpp", []),
]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stdout))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=3) as ex:
        objs = list(ex.map(lambda s: _compile(*s), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stdout))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
