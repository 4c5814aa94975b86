"""GPU parity of chained approximate matvecs: a decode step of a Mistral-7B-shaped
stack (two layers and the output head) and a Mixtral-shaped mixture-of-experts
block.  Every matvec records its parity outputs (the same kernels as the
unrecorded chain, recording on) and is compared with the oracle on the input
vector the GPU actually used (copied back), so the chain's data flow cannot
mask an error: cutoff bits, K, K', per-row kept counts, kept-set fingerprint
and y.  The glue kernels are compared with their plain definitions, and
per-matrix effort schedules run every matvec at its own effort.
"""
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
from _parity import check, rel_l2  # noqa: E402

DIM, KV, HID, VOCAB = 4096, 1024, 14336, 32000
SHAPES = {"wq": (DIM, DIM), "wk": (DIM, KV), "wv": (DIM, KV), "wo": (DIM, DIM),
          "w1": (DIM, HID), "w3": (DIM, HID), "w2": (HID, DIM)}
POOL = ThreadPoolExecutor(min(16, os.cpu_count() or 1))  # the oracle's C calls release the GIL


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_all(jobs, probes):
    """jobs: (key, W, v_used, effort, recorded dict, y_gpu); oracle threaded."""
    def one(job):
        key, W, v, effort, got, y = job
        ref = oracle.run(W, probes[id(W)], np.ascontiguousarray(v, np.float32), effort)
        return key, check(got, ref, where=key, y=y), ref["total_kept"] / W.size
    out = list(POOL.map(one, jobs))
    for key, err, f in out:
        say("  %s rel-L2 %.2e kept %.4f" % (key, err, f))
    return out


def build_stack(d, layers_n):
    Ws, layers = [], []
    for layer in range(layers_n):
        WL, L = {}, {}
        for r in E.LAYER_ROLES:
            m, n = SHAPES[r]
            WL[r] = synth.matrix("config2", m, n, seed=0, layer=layer, w=r)
            L[r] = E.EffortMatrix(WL[r], P=16, device=d)
        Ws.append(WL)
        layers.append(L)
    Wh = synth.matrix("config2", DIM, VOCAB, seed=0, w="head")
    head = E.EffortMatrix(Wh, P=16, device=d)
    to = lambda a: torch.from_numpy(a).to(d)  # noqa: E731
    x = [to(synth.vector("config2/x", DIM, seed=0, layer=l)) for l in range(layers_n)]
    a = [to(synth.vector("config2/attn", DIM, seed=0, layer=l)) for l in range(layers_n)]
    hin = to(synth.vector("config2/head_in", DIM, seed=0))
    probes = {id(W): pr for W, pr in zip(
        [W for WL in Ws for W in WL.values()] + [Wh],
        POOL.map(lambda W: oracle.probes(W, 16), [W for WL in Ws for W in WL.values()] + [Wh]))}
    return Ws, layers, Wh, head, x, a, hin, probes


def step_jobs(step, rec, Ws, Wh, effort, layers_n):
    res = rec.results()
    jobs = []
    for l in range(layers_n):
        ins = {r: t.cpu().numpy() for r, t in step.inputs_of(l).items()}
        for r in E.LAYER_ROLES:
            e = effort(l, r) if callable(effort) else effort
            jobs.append(((l, r), Ws[l][r], ins[r], e, res[(l, r)], step.out[l][r].cpu().numpy()))
    e = effort(None, "head") if callable(effort) else effort
    jobs.append(((None, "head"), Wh, step.head_in.cpu().numpy(), e, res[(None, "head")],
                 step.logits.cpu().numpy()))
    return jobs, res


def test_decode_step_two_layers_and_head():
    d = dev()
    effort = 0.25
    Ws, layers, Wh, head, x, a, hin, probes = build_stack(d, 2)
    step = E.DecodeStep(layers, head, x, a, hin)
    assert step.calls == 15
    # unrecorded eager chain: the reference the recorded and graph runs must reproduce
    step.enqueue(effort)
    torch.cuda.synchronize()
    eager = [{k: v.cpu().numpy().copy() for k, v in o.items()} for o in step.out]
    logits = step.logits.cpu().numpy().copy()

    rec = E.Recorder(d)
    step.enqueue(effort, record=rec)
    jobs, base = step_jobs(step, rec, Ws, Wh, effort, 2)
    for layer in range(2):
        o = step.out[layer]
        assert rel_l2(o["g"].cpu().numpy(), oracle.silu_mul(o["w1"].cpu().numpy(),
                                                            o["w3"].cpu().numpy())) <= 1e-6
        for r in E.LAYER_ROLES:  # recording changes nothing the chain computes
            assert rel_l2(o[r].cpu().numpy(), eager[layer][r]) < 1e-5, (layer, r)
    say("decode step, one stream, every matvec against the oracle:")
    check_all(jobs, probes)

    # side streams and the grouped (multi-matrix) chain, one stream and side
    # streams: every x-fed matvec records exactly the cutoff and kept set of
    # the first run; w2 (whose input depends on fp32 atomics order) against the
    # oracle on its own input
    side = [torch.cuda.Stream() for _ in range(6)]
    gstep = E.DecodeStep(layers, head, x, a, hin, grouped=True)
    for name, st, ss in (("side streams", step, side), ("grouped", gstep, None),
                         ("grouped + side streams", gstep, side)):
        rec2 = E.Recorder(d)
        st.enqueue(effort, side_streams=ss, record=rec2)
        jobs2, res2 = step_jobs(st, rec2, Ws, Wh, effort, 2)
        for job in jobs2:
            key, got = job[0], job[4]
            if key[1] == "w2":
                continue
            ref = base[key]
            assert np.float32(got["cutoff"]).view(np.uint32) == np.float32(ref["cutoff"]).view(np.uint32)
            assert (got["K"], got["Kprime"], got["fingerprint"]) == (ref["K"], ref["Kprime"],
                                                                      ref["fingerprint"]), (name, key)
            assert np.array_equal(got["row_kept"], ref["row_kept"]), (name, key)
        check_all([j for j in jobs2 if j[0][1] == "w2"], probes)
        say("decode step %s: kept sets equal to the one-stream run" % name)

    # the chain captured in a graph replays to the eager result
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step.enqueue(effort)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        step.logits.fill_(float("nan"))
        for o in step.out:
            o["w2"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert rel_l2(step.logits.cpu().numpy(), logits) < 1e-6, rep
        for layer in range(2):
            assert rel_l2(step.out[layer]["w2"].cpu().numpy(), eager[layer]["w2"]) < 1e-5, rep


def test_decode_step_effort_schedule():
    """Every matrix of the step at its own effort (an EffortSchedule), through
    the grouped chain: each matvec against the oracle at that effort."""
    d = dev()
    Ws, layers, Wh, head, x, a, hin, probes = build_stack(d, 2)
    table = [[0.30, 0.20, 0.45, 0.15, 0.25, 0.35, 0.125],
             [0.50, 0.10, 0.22, 0.40, 0.18, 0.27, 0.33]]
    sched = E.EffortSchedule.from_array(table, head=0.2)
    assert sched(1, "wk") == 0.10 and sched(None, "head") == 0.2
    for grouped in (False, True):
        step = E.DecodeStep(layers, head, x, a, hin, grouped=grouped)
        rec = E.Recorder(d)
        step.enqueue(sched, record=rec)
        jobs, res = step_jobs(step, rec, Ws, Wh, sched, 2)
        for (key, W, v, e, got, y) in jobs:
            assert got["K"] == int(np.ceil(np.float64(np.float32(e)) * W.shape[0] * 16)), key
        say("effort schedule (grouped %s):" % grouped)
        check_all(jobs, probes)


def moe_case(d, effort_tag):
    token = int(effort_tag * 100)
    logits = synth.normals(8, seed=token, stream=synth.stream_id("config3/router"))
    route = E.route_top2(logits)
    e0, e1, g0, g1 = route
    experts, Wx = [None] * 8, {}
    for e in (e0, e1):
        Wx[e] = (synth.matrix("config3", DIM, HID, seed=0, expert=e, w="w1"),
                 synth.matrix("config3", DIM, HID, seed=0, expert=e, w="w3"),
                 synth.matrix("config3", HID, DIM, seed=0, expert=e, w="w2"))
        experts[e] = tuple(E.EffortMatrix(W, P=16, device=d) for W in Wx[e])
    x = torch.from_numpy(synth.vector("config3/x", DIM, seed=token)).to(d)
    probes = {id(W): pr for W, pr in zip([W for e in Wx for W in Wx[e]],
                                         POOL.map(lambda W: oracle.probes(W, 16),
                                                  [W for e in Wx for W in Wx[e]]))}
    return route, experts, Wx, x, probes


def moe_jobs(moe, rec, route, Wx, x, effort):
    e0, e1 = route[0], route[1]
    res = rec.results()
    xh = x.cpu().numpy()
    jobs = []
    for k, e in enumerate((e0, e1)):
        W1, W3, W2 = Wx[e]
        h1, h3 = moe.h1[k].cpu().numpy(), moe.h3[k].cpu().numpy()
        gk, ok = moe.g[k].cpu().numpy(), moe.o[k].cpu().numpy()
        assert rel_l2(gk, oracle.silu_mul(h1, h3)) <= 1e-6
        ef = lambda r: effort(e, r) if callable(effort) else effort  # noqa: E731
        jobs += [((e, "w1"), W1, xh, ef("w1"), res[(e, "w1")], h1),
                 ((e, "w3"), W3, xh, ef("w3"), res[(e, "w3")], h3),
                 ((e, "w2"), W2, gk, ef("w2"), res[(e, "w2")], ok)]
    return jobs


@pytest.mark.parametrize("effort", [0.25, 0.16, 0.12])
def test_moe_block_two_routed_experts(effort):
    """Mixtral-shaped block, 8 experts, top-2 routing from seeded logits; only the
    routed experts are materialized (the others are never read).  Ungrouped
    and grouped, one stream and side streams: all six matvecs recorded and
    checked against the oracle, the gated sum against its definition."""
    d = dev()
    route, experts, Wx, x, probes = moe_case(d, effort)
    e0, e1, g0, g1 = route
    say("route", route)
    side = [torch.cuda.Stream() for _ in range(4)]
    for grouped in (False, True):
        moe = E.MoEFFN(experts, d, grouped=grouped)
        for ss in (None, side):
            rec = E.Recorder(d)
            y = moe.enqueue(x, route, effort, side_streams=ss, record=rec)
            jobs = moe_jobs(moe, rec, route, Wx, x, effort)
            check_all(jobs, probes)
            outs = [moe.o[0].cpu().numpy(), moe.o[1].cpu().numpy()]
            y_ref = np.float64(np.float32(g0)) * outs[0] + np.float64(np.float32(g1)) * outs[1]
            assert rel_l2(y.cpu().numpy(), y_ref) <= 1e-6
            say("moe effort %.2f grouped %s side streams %s ok" % (effort, grouped, ss is not None))


def test_moe_block_effort_schedule():
    """Each expert matrix at its own effort: (expert, role) entries and a
    per-role default."""
    d = dev()
    route, experts, Wx, x, probes = moe_case(d, 0.2)
    e0, e1 = route[0], route[1]
    sched = E.EffortSchedule(0.2, {(e0, "w1"): 0.3, (e1, "w3"): 0.14, (None, "w2"): 0.11})
    for grouped in (False, True):
        moe = E.MoEFFN(experts, d, grouped=grouped)
        rec = E.Recorder(d)
        moe.enqueue(x, route, sched, record=rec)
        check_all(moe_jobs(moe, rec, route, Wx, x, sched), probes)


def test_axpby_matches_definition():
    d = dev()
    a = synth.activations(5000, seed=3, stream=11)
    b = synth.activations(5000, seed=4, stream=12)
    out = torch.empty(5000, dtype=torch.float32, device=d)
    E.effort_axpby(torch.from_numpy(a).to(d), 0.625, torch.from_numpy(b).to(d), -1.5, 5000, out)
    torch.cuda.synchronize()
    ref = (np.float32(0.625) * a).astype(np.float32) + (np.float32(-1.5) * b).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
