"""GPU parity of the multi-matrix call (effort_matvec_multi): independent
(matrix, vector) pairs -- matrices sharing one input, or each with its own,
of different heights -- each at its own effort, in one launch per kernel.

Each output must equal the single-matrix call on the same matrix and vector
(the same cutoff and kept set; only the order of the fp32 atomics of the
flush differs, so rel-L2 <= 1e-5 is asked) and lie within rel-L2 1e-3 of the
oracle.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402

SAME_TOL = 1e-5
ORACLE_TOL = 1e-3


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rel_l2(y, ref):
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    d = np.linalg.norm(np.asarray(y, np.float64) - ref)
    return float(d / nr) if nr else float(d)


def run_case(m, ns, efforts, seed, with_oracle=True):
    d = dev()
    Ws = [synth.weights(m, n, seed=seed + j, stream=synth.stream_id("multi", "W", m, n)) for j, n in
          enumerate(ns)]
    v = synth.activations(m, seed=seed, stream=synth.stream_id("multi", "v", m))
    mats = [E.EffortMatrix(W, P=16, device=d) for W in Ws]
    group = E.EffortGroup(mats)
    vt = torch.from_numpy(v).to(d)
    ys = group.matvec(vt, efforts)
    singles = [M.matvec(vt, e) for M, e in zip(mats, efforts)]
    torch.cuda.synchronize()
    print("multi m=%d ns=%s efforts=%s" % (m, ns, efforts), flush=True)
    sys.stdout.flush()
    for j, (W, e) in enumerate(zip(Ws, efforts)):
        y, ys1 = ys[j].cpu().numpy(), singles[j].cpu().numpy()
        assert rel_l2(y, ys1) <= SAME_TOL, (j, rel_l2(y, ys1))
        if with_oracle:
            ref = oracle.run(W, oracle.probes(W, 16), v, e)
            assert rel_l2(y, ref["y"]) <= ORACLE_TOL, (j, rel_l2(y, ref["y"]))
    return ys


@pytest.mark.parametrize("m,ns,efforts", [
    (300, (1000, 257, 64), (0.3, 0.5, 0.125)),
    (256, (256,), (0.25,)),
    (77, (4100, 65), (1.0, 0.01)),
    (513, (2049, 2049, 300, 17), (0.25, 0.25, 0.7, 0.9)),
])
def test_multi_small(m, ns, efforts):
    run_case(m, ns, efforts, seed=5)


def test_multi_mistral_qkv_and_gate_up():
    run_case(4096, (4096, 1024, 1024), (0.25, 0.25, 0.25), seed=11, with_oracle=False)
    run_case(4096, (14336, 14336), (0.25, 0.16), seed=12, with_oracle=False)


def test_multi_repeat_and_reuse():
    # the same group called twice with other efforts: the workspace state of
    # the first call (histograms, counters) must not leak into the second
    d = dev()
    m = 1000
    Ws = [synth.weights(m, n, seed=20 + n, stream=synth.stream_id("multi", "W", m, n)) for n in
          (700, 1300)]
    mats = [E.EffortMatrix(W, P=16, device=d) for W in Ws]
    group = E.EffortGroup(mats)
    for k, efforts in enumerate(((0.25, 0.5), (0.05, 1.0), (0.25, 0.5))):
        v = synth.activations(m, seed=30 + k, stream=synth.stream_id("multi", "v", m))
        vt = torch.from_numpy(v).to(d)
        ys = group.matvec(vt, efforts)
        torch.cuda.synchronize()
        for j, (W, e) in enumerate(zip(Ws, efforts)):
            ref = oracle.run(W, oracle.probes(W, 16), v, e)
            assert rel_l2(ys[j].cpu().numpy(), ref["y"]) <= ORACLE_TOL, (k, j)


def test_multi_own_inputs_and_heights():
    """Pairs with their own vectors and different in_dim (the grid of the chart
    and dispatch kernels is sized by the tallest; the others' extra blocks
    must leave the rest of the workspace alone)."""
    d = dev()
    shapes = [(300, 1000), (2000, 256), (77, 4100), (1024, 64)]
    efforts = [0.25, 0.5, 0.125, 1.0]
    Ws = [synth.weights(m, n, seed=40 + j, stream=synth.stream_id("multi2", "W", m, n))
          for j, (m, n) in enumerate(shapes)]
    vs = [synth.activations(m, seed=50 + j, stream=synth.stream_id("multi2", "v", m))
          for j, (m, n) in enumerate(shapes)]
    mats = [E.EffortMatrix(W, P=16, device=d) for W in Ws]
    group = E.EffortGroup(mats)
    vts = [torch.from_numpy(v).to(d) for v in vs]
    for rep in range(2):
        ys = group.matvec(vts, efforts)
        torch.cuda.synchronize()
        for j, (W, v, e) in enumerate(zip(Ws, vs, efforts)):
            y = ys[j].cpu().numpy()
            y1 = mats[j].matvec(vts[j], e).cpu().numpy()
            assert rel_l2(y, y1) <= SAME_TOL, (rep, j)
            ref = oracle.run(W, oracle.probes(W, 16), v, e)
            assert rel_l2(y, ref["y"]) <= ORACLE_TOL, (rep, j)
        print("multi own inputs rep %d ok" % rep, flush=True)
