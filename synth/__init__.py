"""Seeded synthetic inputs (weights, activations, router logits).

This module only produces numbers; it contains no step of the approximate
multiply.  Both the oracle checks and the GPU path consume exactly the bits it
returns, so generator precision never enters a parity comparison.

Recipe (Philox4x32-10 keyed by splitmix64, Box-Muller in double):
  * weights      W = fp16_rne(0.02 * z)            ~ N(0, 0.02) as fp16 bits
  * activations  v = fp32(0.5 * z0 / sqrt((z1^2+z2^2+z3^2)/3))   Student-t(3)
  * logits       z ~ N(0, 1) in float64
The stream id of an input is a 64-bit FNV-1a hash of a descriptive string
(config, matrix role, layer, expert, vector index), so every input has its own
independent, reproducible stream.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

W_SCALE = 0.02
V_SCALE = 0.5


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i64, u64, f64 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    lib.synth_weights_f16.argtypes = [p, i64, f64, u64, u64]
    lib.synth_student_t3_f32.argtypes = [p, i64, f64, u64, u64]
    lib.synth_normals.argtypes = [p, i64, i64, u64, u64]
    lib.synth_uniforms.argtypes = [p, i64, u64, u64]
    lib.synth_philox4x32_10.argtypes = [p, p, p]
    lib.synth_splitmix64.argtypes = [u64]
    lib.synth_splitmix64.restype = u64
    lib.synth_f64_to_f16.argtypes = [f64]
    lib.synth_f64_to_f16.restype = ctypes.c_uint16
    for f in (lib.synth_weights_f16, lib.synth_student_t3_f32, lib.synth_normals,
              lib.synth_uniforms, lib.synth_philox4x32_10):
        f.restype = None
    _lib = lib
    return lib


def stream_id(*parts) -> int:
    """64-bit FNV-1a of '|'.join(parts): one independent stream per named input."""
    h = 0xCBF29CE484222325
    for b in "|".join(str(p) for p in parts).encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _load().synth_philox4x32_10(c, k, o)
    return tuple(int(x) for x in o)


def splitmix64(x: int) -> int:
    return int(_load().synth_splitmix64(x & 0xFFFFFFFFFFFFFFFF))


def f64_to_f16_bits(x: float) -> int:
    return int(_load().synth_f64_to_f16(float(x)))


def weights(m: int, n: int, seed: int = 0, stream: int = 0, scale: float = W_SCALE) -> np.ndarray:
    """fp16 bits (uint16) of an m x n matrix, row-major, ~ N(0, scale)."""
    out = np.empty((m, n), dtype=np.uint16)
    if out.size:
        _load().synth_weights_f16(out.ctypes.data, out.size, scale, seed, stream)
    return out


def activations(m: int, seed: int = 0, stream: int = 0, scale: float = V_SCALE) -> np.ndarray:
    """fp32 vector of length m ~ scale * Student-t(3)."""
    out = np.empty(m, dtype=np.float32)
    if out.size:
        _load().synth_student_t3_f32(out.ctypes.data, out.size, scale, seed, stream)
    return out


def normals(count: int, seed: int = 0, stream: int = 0, first: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    if count:
        _load().synth_normals(out.ctypes.data, first, count, seed, stream)
    return out


def uniforms(count: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    if count:
        _load().synth_uniforms(out.ctypes.data, count, seed, stream)
    return out


def matrix(role: str, m: int, n: int, seed: int = 0, **tags) -> np.ndarray:
    """Named weight matrix: its stream is derived from the role and the tags."""
    parts = [role, m, n] + ["%s=%s" % kv for kv in sorted(tags.items())]
    return weights(m, n, seed=seed, stream=stream_id(*parts))


def vector(role: str, m: int, seed: int = 0, **tags) -> np.ndarray:
    parts = [role, m] + ["%s=%s" % kv for kv in sorted(tags.items())]
    return activations(m, seed=seed, stream=stream_id(*parts))
