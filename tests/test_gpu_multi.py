"""GPU parity of the multi-matrix call (effort_matvec_multi): independent
(matrix, vector) pairs -- matrices sharing one input, or each with its own,
of different heights -- each at its own effort, in one launch per kernel.

Each pair records its parity outputs (the same kernels and launches with
recording on) and must match the oracle: cutoff bits, K, K', per-row kept
counts, kept-set fingerprint, y within rel-L2 1e-3.  The unrecorded call must
give the single-matrix call's output (the same cutoff and kept set; only the
order of the fp32 atomics of the flush differs, so rel-L2 <= 1e-5 is asked)
and the recorded call's.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from _parity import check  # noqa: E402

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


def recorded(group, vs, efforts):
    """One recorded multi-matrix call: outputs and per-pair parity dicts."""
    rec = E.Recorder(group.mats[0].layout.device)
    ys = group.matvec(vs, efforts, record=(rec, list(range(len(group.mats)))))
    res = rec.results()
    return [y.cpu().numpy() for y in ys], [res[j] for j in range(len(group.mats))]


def run_case(m, ns, efforts, seed):
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
    ys = [y.cpu().numpy() for y in ys]
    yr, got = recorded(group, vt, efforts)
    print("multi m=%d ns=%s efforts=%s" % (m, ns, efforts), flush=True)
    sys.stdout.flush()
    for j, (W, e) in enumerate(zip(Ws, efforts)):
        ys1 = singles[j].cpu().numpy()
        assert rel_l2(ys[j], ys1) <= SAME_TOL, (j, rel_l2(ys[j], ys1))
        assert rel_l2(ys[j], yr[j]) <= SAME_TOL, j
        ref = oracle.run(W, oracle.probes(W, 16), v, e)
        check(got[j], ref, where=("pair", j), y=ys[j])
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
    run_case(4096, (4096, 1024, 1024), (0.25, 0.25, 0.25), seed=11)
    run_case(4096, (14336, 14336), (0.25, 0.16), seed=12)


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
        ys, got = recorded(group, vt, efforts)
        for j, (W, e) in enumerate(zip(Ws, efforts)):
            ref = oracle.run(W, oracle.probes(W, 16), v, e)
            check(got[j], ref, where=(k, j), y=ys[j])


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
        ys = [y.cpu().numpy() for y in group.matvec(vts, efforts)]
        yr, got = recorded(group, vts, efforts)
        for j, (W, v, e) in enumerate(zip(Ws, vs, efforts)):
            y1 = mats[j].matvec(vts[j], e).cpu().numpy()
            assert rel_l2(ys[j], y1) <= SAME_TOL, (rep, j)
            assert rel_l2(ys[j], yr[j]) <= SAME_TOL, (rep, j)
            ref = oracle.run(W, oracle.probes(W, 16), v, e)
            check(got[j], ref, where=(rep, j), y=ys[j])
        print("multi own inputs rep %d ok" % rep, flush=True)


def test_multi_and_batched_many_probes():
    """Pairs with more probes per row than the kernels hold in registers (and
    a mix of probe counts in one call), and batched calls at P = 64 on both
    batch routes (launches of up to 4 vectors; the union pass)."""
    d = dev()
    m = 600
    Ps, ns, efforts = (16, 64, 40), (900, 1300, 700), (0.25, 0.3, 0.6)
    Ws = [synth.weights(m, n, seed=60 + j, stream=synth.stream_id("multiP", "W", m, n))
          for j, n in enumerate(ns)]
    v = synth.activations(m, seed=61, stream=synth.stream_id("multiP", "v", m))
    mats = [E.EffortMatrix(W, P=P, device=d) for W, P in zip(Ws, Ps)]
    group = E.EffortGroup(mats)
    vt = torch.from_numpy(v).to(d)
    ys, got = recorded(group, vt, efforts)
    for j, (W, P, e) in enumerate(zip(Ws, Ps, efforts)):
        check(got[j], oracle.run(W, oracle.probes(W, P), v, e), where=("multi P", P), y=ys[j])
    W = Ws[1]
    M = E.EffortMatrix(W, P=64, device=d, batch=6)
    pr = oracle.probes(W, 64)
    V = np.stack([synth.activations(m, seed=70 + s, stream=synth.stream_id("multiP", "v")) for s in range(6)])
    for effort, b in ((0.25, 3), (0.8, 6)):
        res = M.matvec_batched_debug(torch.from_numpy(V[:b]).to(d), effort)
        for k in range(b):
            check(res[k], oracle.run(W, pr, V[k], effort), where=("batched P=64", effort, b, k))
    print("multi and batched with many probes ok", flush=True)


def test_multi_and_batched_thirty_two_probes():
    """P = 32 pairs in one multi-matrix call (the 8-lane dispatch for all), a
    call mixing P = 32 with P = 16 (the row-per-thread dispatch for all), and
    batched P = 32 calls on both batch routes."""
    d = dev()
    m = 1500
    Ws = [synth.weights(m, n, seed=80 + j, stream=synth.stream_id("multi32", "W", m, n))
          for j, n in enumerate((900, 2100, 700))]
    v = synth.activations(m, seed=81, stream=synth.stream_id("multi32", "v", m))
    vt = torch.from_numpy(v).to(d)
    for Ps, efforts in (((32, 32, 32), (0.25, 0.1, 0.7)), ((32, 16, 32), (0.3, 0.3, 0.05))):
        mats = [E.EffortMatrix(W, P=P, device=d) for W, P in zip(Ws, Ps)]
        group = E.EffortGroup(mats)
        ys, got = recorded(group, vt, efforts)
        for j, (W, P, e) in enumerate(zip(Ws, Ps, efforts)):
            check(got[j], oracle.run(W, oracle.probes(W, P), v, e), where=("multi", Ps, j), y=ys[j])
    W = Ws[1]
    M = E.EffortMatrix(W, P=32, device=d, batch=6)
    pr = oracle.probes(W, 32)
    V = np.stack([synth.activations(m, seed=90 + s, stream=synth.stream_id("multi32", "v")) for s in range(6)])
    for effort, b in ((0.25, 3), (0.25, 6), (0.8, 6)):
        res = M.matvec_batched_debug(torch.from_numpy(V[:b]).to(d), effort)
        for k in range(b):
            check(res[k], oracle.run(W, pr, V[k], effort), where=("batched P=32", effort, b, k))
    print("multi and batched with 32 probes ok", flush=True)
