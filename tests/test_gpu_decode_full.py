"""Parity of a Mistral-7B-shaped decode step: layers of 7 matrices plus the
4096x32000 head at effort 0.25, random-init seeded weights,
run through the grouped chain (the multi-matrix calls for (wq, wk, wv) and
(w1, w3)) with every matvec recording its parity outputs.  Every matvec is
checked against the oracle on the input the GPU actually used (w2's input is
formed from the approximate h1 and h3): cutoff bits, K, K', per-row kept
counts, kept-set fingerprint, and y within rel-L2 1e-3; the unrecorded chain
gives the recorded chain's outputs.  The oracle runs in a thread pool (its C calls release the GIL);
the weights are regenerated from their seeds for the check, not kept.
EFFORT_DECODE_LAYERS sets the number of layers: 8 by default (57 matvecs, about
a minute with the oracle's probe sorts), 32 for the whole step (225 matvecs,
several minutes of host CPU)."""
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
from _parity import check  # noqa: E402

DIM, KV, HID, VOCAB = 4096, 1024, 14336, 32000
SHAPES = {"wq": (DIM, DIM), "wk": (DIM, KV), "wv": (DIM, KV), "wo": (DIM, DIM),
          "w1": (DIM, HID), "w3": (DIM, HID), "w2": (HID, DIM)}
LAYERS = int(os.environ.get("EFFORT_DECODE_LAYERS", "8"))
REL_L2_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(y, ref):
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(y, np.float64) - ref) / nr) if nr else 0.0


def test_full_decode_step_every_matvec():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda:0")
    effort = 0.25
    layers = []
    for l in range(LAYERS):
        layers.append({r: E.EffortMatrix(synth.matrix("config2", m, n, seed=0, layer=l, w=r), P=16,
                                         device=d) for r, (m, n) in SHAPES.items()})
        if l % 8 == 7:
            say("layers prepared: %d" % (l + 1))
    head = E.EffortMatrix(synth.matrix("config2", DIM, VOCAB, seed=0, w="head"), P=16, device=d)
    to = lambda a: torch.from_numpy(a).to(d)  # noqa: E731
    x = [to(synth.vector("config2/x", DIM, seed=0, layer=l)) for l in range(LAYERS)]
    a = [to(synth.vector("config2/attn", DIM, seed=0, layer=l)) for l in range(LAYERS)]
    hin = to(synth.vector("config2/head_in", DIM, seed=0))
    step = E.DecodeStep(layers, head, x, a, hin, grouped=True)
    assert step.calls == 7 * LAYERS + 1
    step.enqueue(effort)  # unrecorded
    torch.cuda.synchronize()
    plain = {(l, r): step.out[l][r].cpu().numpy().copy() for l in range(LAYERS) for r in E.LAYER_ROLES}
    plain[(None, "head")] = step.logits.cpu().numpy().copy()
    rec = E.Recorder(d)
    step.enqueue(effort, record=rec)
    res = rec.results()
    say("decode step ran: %d matvecs, %d recorded" % (step.calls, len(res)))
    assert len(res) == step.calls

    jobs = []
    for l in range(LAYERS):
        ins = {r: t.cpu().numpy() for r, t in step.inputs_of(l).items()}
        for r in E.LAYER_ROLES:
            y = step.out[l][r].cpu().numpy()
            if r != "w2":  # x-fed: the same input as the unrecorded run
                assert rel_l2(y, plain[(l, r)]) < 1e-5, (l, r)
            jobs.append((("config2", SHAPES[r], l, r), ins[r], y, res[(l, r)]))
    jobs.append((("config2", (DIM, VOCAB), None, "head"), hin.cpu().numpy(),
                 step.logits.cpu().numpy(), res[(None, "head")]))
    assert rel_l2(step.logits.cpu().numpy(), plain[(None, "head")]) < 1e-5

    def one(job):
        (cfg, (m, n), l, r), v, y, got = job
        W = (synth.matrix(cfg, m, n, seed=0, layer=l, w=r) if l is not None
             else synth.matrix(cfg, m, n, seed=0, w=r))
        ref = oracle.run(W, oracle.probes(W, 16), np.ascontiguousarray(v, np.float32), effort)
        try:
            return (l, r), check(got, ref, where=(l, r), y=y), None
        except AssertionError as exc:
            return (l, r), float("inf"), exc

    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        results = list(ex.map(one, jobs))
    bad = [(k, exc) for k, e, exc in results if exc is not None]
    assert not bad, bad[:5]
    worst = max(results, key=lambda t: t[1])
    say("%d matvecs checked (cutoff, K, K', kept set, y), worst rel-L2 %.2e at %s" % (
        len(results), worst[1], worst[0]))
