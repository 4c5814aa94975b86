"""Parity over the whole benchmark sweep: the four Mistral-7B-shaped matrices
(4096x4096, 4096x1024, 4096x14336, 14336x4096, P = 16, default groups), 100
seeded vectors each, at effort 1, 0.5, 0.25 and 0.125 -- 1600 points.  On every
point: cutoff bits, K, K', per-row kept counts and the kept-set fingerprint
equal to the oracle's, y within rel-L2 1e-3.  Over the oracle's results it also
checks the kept-fraction bound (effort <= f <= K'/N + (ceil(n/P) - 1)/n, the
bound of the end-of-segment probes) and reports f per effort, and that the
error against effort 1 does not decrease as the effort drops (per vector, and
for the mean).

The oracle costs about a second of host CPU per point; threaded over the
host's cores the whole sweep takes under a minute on the GPU host.
EFFORT_PARITY_SWEEP_VECTORS sets the number of vectors (default 100).
"""
import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402

REL_L2_TOL = 1e-3
SHAPES = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)]
EFFORTS = (1.0, 0.5, 0.25, 0.125)
NV = int(os.environ.get("EFFORT_PARITY_SWEEP_VECTORS", "100"))
P = 16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(y, ref):
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(y, np.float64) - ref) / nr) if nr else 0.0


@pytest.mark.parametrize("shape", SHAPES)
def test_sweep(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda:0")
    m, n = shape
    W = synth.matrix("config1", m, n, seed=0)
    M = E.EffortMatrix(W, P=P, device=d)
    V = [synth.vector("config1", m, seed=s) for s in range(NV)]
    say("sweep %dx%d: %d vectors x %d efforts on the GPU" % (m, n, NV, len(EFFORTS)))
    got = {}
    for s in range(NV):
        vt = torch.from_numpy(V[s]).to(d)
        for e in EFFORTS:
            got[(s, e)] = M.matvec_debug(vt, e, with_mask=False)
    say("sweep %dx%d: oracle" % (m, n))
    pr = oracle.probes(W, P)
    keys = list(got)
    workers = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:  # the oracle's C calls release the GIL
        refs = dict(zip(keys, ex.map(lambda k: oracle.run(W, pr, V[k[0]], k[1]), keys)))

    N = m * P
    slack = (math.ceil(n / P) - 1) / n
    worst = 0.0
    frac = {e: [] for e in EFFORTS}
    for k in keys:
        g, r = got[k], refs[k]
        where = "%dx%d seed %d effort %g" % (m, n, k[0], k[1])
        assert np.float32(g["cutoff"]).view(np.uint32) == np.float32(r["cutoff"]).view(np.uint32), where
        assert g["K"] == r["K"] and g["Kprime"] == r["Kprime"], where
        assert np.array_equal(g["row_kept"], r["row_kept"]), where
        assert g["fingerprint"] == r["fingerprint"], where
        err = rel_l2(g["y"], r["y"])
        assert err <= REL_L2_TOL, (where, err)
        worst = max(worst, err)
        f = r["total_kept"] / (m * n)
        assert k[1] <= f + 1e-12 and f <= r["Kprime"] / N + slack + 1e-12, (where, f)
        frac[k[1]].append(f)
    # error against effort 1 does not shrink as the effort drops
    errs = np.array([[np.linalg.norm(refs[(s, e)]["y"] - refs[(s, 1.0)]["y"]) for e in EFFORTS]
                     for s in range(NV)])
    assert np.all(np.diff(errs, axis=1) >= 0.0), "a vector whose error shrinks as the effort drops"
    assert np.all(np.diff(errs.mean(axis=0)) >= 0.0)
    say("sweep %dx%d: %d points equal, worst rel-L2 %.2e; kept fraction %s" % (
        m, n, len(keys), worst,
        ", ".join("%g: %.4f (%.4f..%.4f)" % (e, np.mean(frac[e]), np.min(frac[e]), np.max(frac[e]))
                  for e in EFFORTS)))
