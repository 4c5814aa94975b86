"""MI355X (gfx950) implementation of the "Effort" approximate vector-matrix multiply.

The compute path is libeffort.so (hand-written HIP kernels behind the C ABI of
include/effort.h).  This package is its ctypes binding, a small holder for a
prepared matrix resident in device memory, and the sequencing of chained calls
(a decoder stack's matvecs, a mixture-of-experts block); PyTorch only supplies
device memory and streams.
"""
from .binding import *  # noqa: F401,F403
from .binding import EffortError, effort_desc, LIB_PATH  # noqa: F401
from .chain import (LAYER_ROLES, DecodeStep, DenseDecodeStep, EffortSchedule, MoEFFN,  # noqa: F401
                    route_top2)
from .device import EffortGroup, EffortMatrix, Recorder  # noqa: F401

__all__ = [n for n in dir() if n.startswith(("effort_", "dense_")) or n in
           ("EffortError", "EffortGroup", "EffortMatrix", "LIB_PATH", "LAYER_ROLES", "DecodeStep",
            "DenseDecodeStep", "EffortSchedule", "MoEFFN", "Recorder", "route_top2")]
