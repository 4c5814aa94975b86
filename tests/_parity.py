"""The parity contract shared by the GPU tests: the cutoff bit-equal (uint32
pattern), K and K' equal, the kept set equal (per-row kept counts and the
order-free 64-bit fingerprint, plus the uint8 mask where the case records it)
and y within rel-L2 1e-3 of the oracle's double-precision sums (if the
oracle's y is exactly zero, |y_gpu| <= 1e-30)."""
import numpy as np

REL_L2_TOL = 1e-3


def rel_l2(y, ref):
    ref = np.asarray(ref, np.float64)
    y = np.asarray(y, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.max(np.abs(y), initial=0.0) <= 1e-30 else np.inf
    return float(np.linalg.norm(y - ref) / nr)


def check_kept(got, ref, where=""):
    """Cutoff bits, K, K', per-row kept counts and fingerprint."""
    assert np.float32(got["cutoff"]).view(np.uint32) == np.float32(ref["cutoff"]).view(np.uint32), \
        (where, got["cutoff"], ref["cutoff"])
    assert got["K"] == ref["K"] and got["Kprime"] == ref["Kprime"], \
        (where, got["K"], ref["K"], got["Kprime"], ref["Kprime"])
    assert np.array_equal(np.asarray(got["row_kept"], np.int64), ref["row_kept"]), where
    assert got["fingerprint"] == ref["fingerprint"], where


def check(got, ref, with_mask=False, where="", y=None):
    """The whole contract; `y` overrides got["y"] (an output recorded elsewhere)."""
    check_kept(got, ref, where)
    if with_mask:
        assert np.array_equal(got["mask"], ref["mask"]), where
    err = rel_l2(got["y"] if y is None else y, ref["y"])
    assert err <= REL_L2_TOL, (where, err)
    return err
