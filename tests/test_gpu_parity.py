"""GPU parity: libeffort against the oracle on the same seeded inputs.

Contract checked on every case:
  * cutoff bit-equal (uint32 pattern), K and K' equal;
  * kept set equal: per-row kept counts and the 64-bit order-free fingerprint,
    plus the full uint8 mask where the case says so;
  * y within rel-L2 <= 1e-3 of the oracle's double-precision sums (the GPU
    accumulates in fp32 with atomics in no fixed order); if the oracle's y is
    exactly zero, |y_gpu| <= 1e-30.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

REL_L2_TOL = 1e-3

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from _parity import check, rel_l2  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()




def case(m, n, seed, tag):
    W = synth.weights(m, n, seed=seed, stream=synth.stream_id(tag, "W", m, n))
    v = synth.activations(m, seed=seed, stream=synth.stream_id(tag, "v", m))
    return W, v


def run_pair(W, v, P, effort, groups=0, with_mask=True, where=""):
    d = dev()
    M = E.EffortMatrix(W, P=P, groups=groups, device=d)
    vt = torch.from_numpy(np.ascontiguousarray(v)).to(d)
    got = M.matvec_debug(vt, effort, with_mask=with_mask)
    ref = oracle.run(W, oracle.probes(W, P), v, effort, mask=with_mask)
    return check(got, ref, with_mask, where)


# ---------------------------------------------------------------- small cases (full mask)

def test_hand_example():
    import json
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    W = np.array(g["W"], dtype=np.float16).view(np.uint16)
    v = np.array(g["v"], dtype=np.float32)
    M = E.EffortMatrix(W, P=g["P"], device=dev())
    vt = torch.from_numpy(v).to(dev())
    for c in g["cases"]:
        got = M.matvec_debug(vt, c["effort"])
        assert float(got["cutoff"]) == c["cutoff"]
        assert got["K"] == c["K"] and got["Kprime"] == c["Kprime"]
        assert got["mask"].tolist() == c["mask"]
        assert np.allclose(got["y"], c["y"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("P", [16, 1, 256])
@pytest.mark.parametrize("effort", [1.0, 0.5, 0.25])
def test_config0(P, effort):
    """256 x 256, W ~ N(0, 0.02) fp16, v ~ 0.5 Student-t(3), seed 0."""
    W = synth.matrix("config0", 256, 256, seed=0)
    v = synth.vector("config0", 256, seed=0)
    say("config0 P=%d effort=%g" % (P, effort))
    run_pair(W, v, P, effort, where="config0")


@pytest.mark.parametrize("m,n,P,G", [(300, 1000, 16, 0), (1, 1, 1, 0), (7, 65, 3, 2),
                                     (513, 2049, 16, 3), (64, 8192, 8, 1), (100, 100, 100, 0),
                                     (2, 5000, 5, 0), (1000, 3, 2, 0), (257, 300, 16, 5),
                                     (600, 4000, 16, 8), (1000, 9000, 16, 6)])
@pytest.mark.parametrize("effort", [0.05, 0.3, 1.0])
def test_ragged_shapes(m, n, P, G, effort):
    W, v = case(m, n, seed=m + n, tag="ragged")
    say("ragged m=%d n=%d P=%d G=%d effort=%g" % (m, n, P, G, effort))
    run_pair(W, v, P, effort, groups=G, where="ragged")


@pytest.mark.parametrize("m,n,G,fmt", [(700, 3000, 0, 0), (2048, 1100, 3, 1), (2049, 4100, 8, 0),
                                        (3000, 5000, 0, 1), (33, 70, 1, 0)])
@pytest.mark.parametrize("effort", [0.02, 0.25, 1.0])
def test_thirty_two_probes(m, n, G, fmt, effort):
    """P = 32 takes the dispatch with 8 lanes per row (32 rows per block): its
    candidates in per-block regions up to 2048 rows (64 blocks), in one list
    beyond; every group count up to 8 and a ragged last block."""
    d = dev()
    W, v = case(m, n, seed=m + n + 32, tag="p32")
    M = E.EffortMatrix(W, P=32, groups=G, device=d, entry_format=fmt)
    vt = torch.from_numpy(v).to(d)
    got = M.matvec_debug(vt, effort, with_mask=m * n <= (1 << 24))
    ref = oracle.run(W, oracle.probes(W, 32), v, effort, mask=got["mask"] is not None)
    check(got, ref, got["mask"] is not None, where=("P=32", m, n, G, fmt, effort))
    y = M.matvec(vt, effort)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), got["y"]) < 1e-6
    say("P=32 %dx%d G=%d format %d effort %g ok" % (m, n, M.groups, fmt, effort))


@pytest.mark.parametrize("P", [33, 40, 64, 100, 300])
@pytest.mark.parametrize("effort", [0.02, 0.25, 1.0])
def test_many_probes(P, effort):
    """More probes per row than the kernels hold in registers (32): the chart
    and dispatch read them in chunks of 32 keys (16-byte loads when P is a
    multiple of 8), with a partial last chunk."""
    W, v = case(700, 3000, seed=P, tag="manyp")
    say("many probes P=%d effort=%g" % (P, effort))
    run_pair(W, v, P, effort, where=("many probes", P, effort))


@pytest.mark.parametrize("m,n,G", [(4097, 512, 0), (5000, 700, 3), (9000, 1024, 8), (14336, 300, 2),
                                   (40000, 256, 0), (70000, 128, 0)])
def test_tall_matrices(m, n, G):
    """Tall matrices, whose dispatch blocks (more than 64) put the cutoff's
    candidates in one list instead of per-block regions: single and batched
    calls against the oracle, from just past 4096 rows to 70000."""
    W, v = case(m, n, seed=m + n, tag="tall")
    for effort in (0.01, 0.25, 1.0):
        say("tall m=%d n=%d G=%d effort=%g" % (m, n, G, effort))
        run_pair(W, v, 16, effort, groups=G, with_mask=m * n <= (1 << 22), where=("tall", m, n, effort))
    d = dev()
    M = E.EffortMatrix(W, P=16, groups=G, device=d, batch=6)
    V = np.stack([case(m, n, seed=m + n + 1 + k, tag="tallv")[1] for k in range(6)])
    pr = oracle.probes(W, 16)
    got = M.matvec_batched_debug(torch.from_numpy(V).to(d), 0.25)
    for k in range(6):
        check(got[k], oracle.run(W, pr, V[k], 0.25), where=("tall batched", m, n, k))


@pytest.mark.parametrize("fmt", [E.EFFORT_ENTRY_U32, E.EFFORT_ENTRY_R12])
def test_extreme_activation_scales(fmt):
    """Activations far from unit scale: the tile's fixed-point scale comes from
    the bound sum |v_i| rowmax_i, so v scaled by 1e30 or 1e-30 (chart values
    near fp32 denormals) and a vector mixing 1e15 and 1e-15 keep the oracle's
    cutoff, kept set and y.  (|v| 1e30 times the largest fp16 stays finite.)"""
    d = dev()
    W, v = case(500, 1200, seed=13, tag="scales")
    mixed = v.copy()
    mixed[::2] *= 1e15
    mixed[1::2] *= 1e-15
    M = E.EffortMatrix(W, P=16, device=d, entry_format=fmt)
    pr = oracle.probes(W, 16)
    for name, vs in (("1e30", v * np.float32(1e30)), ("1e-30", v * np.float32(1e-30)), ("mixed", mixed)):
        vs = np.ascontiguousarray(vs, np.float32)
        assert np.all(np.isfinite(vs))
        vt = torch.from_numpy(vs).to(d)
        for effort in (0.3, 1.0):
            got = M.matvec_debug(vt, effort, with_mask=True)
            ref = oracle.run(W, pr, vs, effort, mask=True)
            check(got, ref, True, where=("scales", name, effort, fmt))
            y = M.matvec(vt, effort)
            torch.cuda.synchronize()
            assert rel_l2(y.cpu().numpy(), ref["y"]) <= REL_L2_TOL, (name, effort)
            say("scale %s effort %g format %d ok" % (name, effort, fmt))


def test_degenerate_inputs():
    d = dev()
    # zero vector: cutoff 0 keeps everything, y = 0
    W, v = case(64, 200, seed=1, tag="degen")
    run_pair(W, np.zeros(64, np.float32), 8, 0.25, where="zero v")
    # equal magnitudes everywhere: whole rows tie
    We = np.full((32, 96), np.float16(0.5).view(np.uint16), np.uint16)
    We[::3] |= 0x8000
    run_pair(We, np.linspace(-2, 2, 32).astype(np.float32), 4, 0.3, where="ties")
    # fp16 subnormal and zero weights
    Ws = W.copy()
    Ws[:, ::2] &= 0x83FF
    Ws[:, 1::7] = 0
    run_pair(Ws, v, 8, 0.4, where="subnormal")
    # one dominant activation, tiny effort (K = 1)
    v2 = v.copy() * 1e-3
    v2[5] = 40.0
    run_pair(W, v2, 8, 1e-7, where="K=1")
    # activations that are exactly zero in some rows
    v3 = v.copy()
    v3[::2] = 0.0
    run_pair(W, v3, 16, 0.5, where="zero rows")
    del d


def test_debug_flags_nonfinite_activations():
    """A NaN or an infinity in v is outside the contract; the debug entry point
    reports it (bit 0 of its status word) and reports nothing for finite v."""
    W, v = case(300, 700, seed=5, tag="finite")
    M = E.EffortMatrix(W, P=16, device=dev())
    assert not M.matvec_debug(torch.from_numpy(v).to(dev()), 0.25, with_mask=False)["v_nonfinite"]
    for bad in (np.float32("nan"), np.float32("inf"), np.float32("-inf")):
        vb = v.copy()
        vb[123] = bad
        got = M.matvec_debug(torch.from_numpy(vb).to(dev()), 0.25, with_mask=False)
        assert got["v_nonfinite"], bad
    # the flag does not stick: the next finite call clears it
    assert not M.matvec_debug(torch.from_numpy(v).to(dev()), 0.25, with_mask=False)["v_nonfinite"]


def test_repeat_calls_and_workspace_reuse():
    W, v = case(512, 3000, seed=3, tag="repeat")
    M = E.EffortMatrix(W, P=16, device=dev())
    vt = torch.from_numpy(v).to(dev())
    a = M.matvec_debug(vt, 0.25)
    b = M.matvec_debug(vt, 1.0)
    c = M.matvec_debug(vt, 0.25)
    assert np.float32(a["cutoff"]) == np.float32(c["cutoff"])
    assert np.array_equal(a["mask"], c["mask"]) and a["fingerprint"] == c["fingerprint"]
    assert b["total_kept"] == W.size
    assert rel_l2(a["y"], c["y"]) < 1e-6
    # the timed entry point (no recording) gives the same y
    y = M.matvec(vt, 0.25)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), a["y"]) < 1e-6


def test_batched_matches_single_vectors():
    d = dev()
    W = synth.matrix("batched", 1024, 2048, seed=0)
    M = E.EffortMatrix(W, P=16, device=d, batch=5)
    V = np.stack([synth.vector("batched", 1024, seed=s) for s in range(5)])
    Vt = torch.from_numpy(V).to(d)
    Y = M.matvec_batched(Vt, 0.25)
    torch.cuda.synchronize()
    got = M.matvec_batched_debug(Vt, 0.25, with_mask=True)
    pr = oracle.probes(W, 16)
    for b in range(5):
        ref = oracle.run(W, pr, V[b], 0.25, mask=True)
        check(got[b], ref, with_mask=True, where=("batched", b))
        assert rel_l2(Y[b].cpu().numpy(), got[b]["y"]) < 1e-6
        single = M.matvec_debug(Vt[b].contiguous(), 0.25, with_mask=False)
        assert single["fingerprint"] == got[b]["fingerprint"]


# ---------------------------------------------------------------- comparators and glue

@pytest.mark.parametrize("m,n", [(256, 256), (4096, 1024), (300, 1001), (1, 8), (77, 4100),
                                 (4096, 14336), (14336, 4096), (4096, 32000), (513, 2048), (5, 16384)])
def test_dense_gemv(m, n):
    d = dev()
    W, v = case(m, n, seed=7, tag="dense")
    Wt = torch.from_numpy(W.view(np.int16)).to(d)
    y = torch.empty(n, dtype=torch.float32, device=d)
    E.dense_gemv(Wt, torch.from_numpy(v).to(d), m, n, y)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), oracle.dense(W, v)) <= 1e-5


@pytest.mark.parametrize("b", [1, 2, 3, 5, 16])
def test_dense_gemm_small(b):
    d = dev()
    m, n = 512, 1100
    W = synth.matrix("gemm", m, n, seed=0)
    V = np.stack([synth.vector("gemm", m, seed=s) for s in range(b)])
    Y = torch.empty((b, n), dtype=torch.float32, device=d)
    E.dense_gemm_small(torch.from_numpy(W.view(np.int16)).to(d), torch.from_numpy(V).to(d), b, m, n, Y)
    torch.cuda.synchronize()
    for i in range(b):
        assert rel_l2(Y[i].cpu().numpy(), oracle.dense(W, V[i])) <= 1e-5


def test_silu_mul():
    d = dev()
    h1 = synth.activations(10000, seed=1, stream=5) * 4
    h3 = synth.activations(10000, seed=2, stream=6)
    out = torch.empty(10000, dtype=torch.float32, device=d)
    E.effort_silu_mul(torch.from_numpy(h1).to(d), torch.from_numpy(h3).to(d), 10000, out)
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), oracle.silu_mul(h1, h3)) <= 1e-6


# ---------------------------------------------------------------- Mistral-7B-shaped matrices

SHAPES = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)]
_probe_cache = {}


@pytest.mark.parametrize("shape", SHAPES)
def test_mistral_shapes(shape):
    """Full-size matrices in the configuration the benchmark times (P = 16,
    default groups): every effort of the sweep on seeds 0-4, the full uint8
    mask compared on every point."""
    from concurrent.futures import ThreadPoolExecutor

    d = dev()
    m, n = shape
    W = synth.matrix("config1", m, n, seed=0)
    say("shape %dx%d: oracle probes" % (m, n))
    pr = oracle.probes(W, 16)
    M = E.EffortMatrix(W, P=16, device=d)
    pts = [(seed, effort) for seed in range(5) for effort in (1.0, 0.5, 0.25, 0.125)]
    V = {seed: synth.vector("config1", m, seed=seed) for seed in range(5)}
    with ThreadPoolExecutor(4) as ex:  # the oracle's C calls release the GIL
        for (seed, effort), ref in zip(pts, ex.map(lambda p: oracle.run(W, pr, V[p[0]], p[1], mask=True),
                                                    pts)):
            got = M.matvec_debug(torch.from_numpy(V[seed]).to(d), effort, with_mask=True)
            err = check(got, ref, True, where="%dx%d/%d/%g" % (m, n, seed, effort))
            say("shape %dx%d seed %d effort %g ok kept=%.4f relL2=%.2e" % (
                m, n, seed, effort, ref["total_kept"] / W.size, err))


@pytest.mark.parametrize("fmt", [E.EFFORT_ENTRY_R12, E.EFFORT_ENTRY_U32])
def test_headline_timed_entry_several_seeds(fmt):
    """The benchmarked entry point itself (effort_matvec, no recording) at
    4096x14336, effort 0.25, seeds 0-4, on the layout the benchmark times (r12
    entries) and the 4-byte one: its cutoff bits, K and K' (the result words
    it leaves in the workspace) and y against the oracle; the recording entry
    point on the same input (the same kernels, recording on) gives the same y
    and the oracle's kept set, fingerprint and full mask."""
    d = dev()
    m, n, effort = 4096, 14336, 0.25
    W = synth.matrix("config1", m, n, seed=0)
    pr = oracle.probes(W, 16)
    M = E.EffortMatrix(W, P=16, device=d, entry_format=fmt)
    for seed in range(5):
        v = synth.vector("config1", m, seed=seed)
        vt = torch.from_numpy(v).to(d)
        ref = oracle.run(W, pr, v, effort, mask=True)
        y = M.matvec(vt, effort)
        torch.cuda.synchronize()
        res = M.ws[:16].cpu().numpy().view(np.uint32)
        assert res[0] == np.float32(ref["cutoff"]).view(np.uint32), seed
        assert res[2] == ref["K"] and res[1] == ref["Kprime"], seed
        y = y.cpu().numpy()
        assert rel_l2(y, ref["y"]) <= REL_L2_TOL, seed
        got = M.matvec_debug(vt, effort, with_mask=True)
        check(got, ref, True, where=("headline", seed))
        assert rel_l2(got["y"], y) < 1e-6, seed
        say("headline format %d seed %d: timed entry and recording entry equal the oracle" % (fmt, seed))


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph give the eager result on every replay
    (with eager work and synchronizations between replays)."""
    d = dev()
    W, v = case(1024, 4096, seed=9, tag="graph")
    M = E.EffortMatrix(W, P=16, device=d)
    vt = torch.from_numpy(v).to(d)
    ref = M.matvec_debug(vt, 0.25)
    y = torch.empty(4096, dtype=torch.float32, device=d)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            E.effort_matvec(M.desc, M.layout, vt, 0.25, y, M.ws, M.ws_bytes)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(5):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert rel_l2(y.cpu().numpy(), ref["y"]) < 1e-6, rep
        # eager work between replays, on the same workspace
        other = M.matvec_debug(vt, 0.5 if rep % 2 else 0.25, with_mask=False)
        assert other["K"] > 0


def test_graph_replays_multi_and_batched():
    """A multi-matrix call and batched calls on both routes (launches of up to
    4 vectors at effort 0.25, the union pass at 0.8), captured in one HIP
    graph, give their eager results on every replay, with eager calls on the
    same workspaces between the replays."""
    d = dev()
    W1, v = case(1024, 3000, seed=21, tag="graphm")
    W2, _ = case(1024, 1100, seed=22, tag="graphm")
    M1 = E.EffortMatrix(W1, P=16, device=d, batch=6)
    M2 = E.EffortMatrix(W2, P=16, device=d)
    group = E.EffortGroup([M1, M2])
    vt = torch.from_numpy(v).to(d)
    V = torch.from_numpy(np.stack([case(1024, 8, seed=30 + k, tag="graphv")[1] for k in range(6)])).to(d)
    ys = [torch.empty(3000, dtype=torch.float32, device=d), torch.empty(1100, dtype=torch.float32, device=d)]
    Yb = {e: torch.empty((6, 3000), dtype=torch.float32, device=d) for e in (0.25, 0.8)}
    # eager references (the batched ones on the layout's own workspace)
    ref_multi = [y.cpu().numpy() for y in group.matvec(vt, [0.25, 0.4])]
    ref_b = {e: M1.matvec_batched(V, e).cpu().numpy() for e in (0.25, 0.8)}
    torch.cuda.synchronize()

    def work():
        group.matvec(vt, [0.25, 0.4], ys=ys)
        for e in (0.25, 0.8):
            M1.matvec_batched(V, e, y=Yb[e])

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys + list(Yb.values()):
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for j in range(2):
            assert rel_l2(ys[j].cpu().numpy(), ref_multi[j]) < 1e-5, (rep, j)
        for e in (0.25, 0.8):
            got = Yb[e].cpu().numpy()
            for k in range(6):
                assert rel_l2(got[k], ref_b[e][k]) < 1e-5, (rep, e, k)
        # eager calls between replays, on the same workspaces
        group.matvec(vt, [0.05, 1.0])
        M1.matvec_batched(V[:3], 0.5)
        torch.cuda.synchronize()
    say("graph replays of multi and batched calls match eager")


def test_timed_entry_matches_and_stamps_kernels():
    """effort_matvec_timed gives the untimed result and a positive duration for
    each of its three kernels; a half-set event pair is rejected."""
    d = dev()
    W, v = case(2048, 4096, seed=11, tag="timed")
    M = E.EffortMatrix(W, P=16, device=d)
    vt = torch.from_numpy(v).to(d)
    ref = M.matvec_debug(vt, 0.25, with_mask=False)
    y = torch.empty(4096, dtype=torch.float32, device=d)
    evs = [E.effort_event_create() for _ in range(6)]
    try:
        for _ in range(3):
            E.effort_matvec_timed(M.desc, M.layout, vt, 0.25, y, M.ws, M.ws_bytes, evs)
            torch.cuda.synchronize()
            assert rel_l2(y.cpu().numpy(), ref["y"]) < 1e-6
            for k in range(3):
                ms = E.effort_event_elapsed_ms(evs[2 * k], evs[2 * k + 1])
                assert 0.0 < ms < 100.0, (k, ms)
        with pytest.raises(E.EffortError):
            E.effort_matvec_timed(M.desc, M.layout, vt, 0.25, y, M.ws, M.ws_bytes,
                                  [evs[0], None, None, None, None, None])
    finally:
        torch.cuda.synchronize()
        for e in evs:
            E.effort_event_destroy(e)


@pytest.mark.parametrize("m,n", [(20000, 300), (70000, 64)])
def test_many_rows_few_columns(m, n):
    """Tall matrices with a narrow output (one column group): 79 and 274 blocks
    of 256 rows; above 256 the multiply sums the per-block read lengths in more
    than one round and locates a share's first block in global memory."""
    W, v = case(m, n, seed=22, tag="tall")
    say("tall m=%d n=%d" % (m, n))
    run_pair(W, v, 16, 0.25, with_mask=False, where="tall")


@pytest.mark.parametrize("m,n,G,b,P,effort", [(4096, 14336, 0, 2, 16, 0.25), (4096, 14336, 0, 9, 16, 0.25),
                                              (4096, 14336, 0, 16, 16, 0.75), (4096, 14336, 0, 9, 16, 1.0),
                                              (513, 2049, 3, 3, 16, 0.25), (300, 1000, 0, 16, 5, 0.25),
                                              (300, 1000, 0, 16, 5, 0.8), (64, 8192, 1, 4, 8, 0.25),
                                              (513, 2049, 3, 7, 16, 0.1), (300, 1000, 0, 16, 5, 0.5),
                                              (513, 2049, 3, 6, 16, 1.0)])
def test_batched_fused_matches_oracle(m, n, G, b, P, effort):
    """Batched calls (up to 4 vectors, or any number below effort 0.625:
    launches of up to 4 vectors, each with its own multiply; from 5 vectors at
    effort 0.625 and above: passes of up to 8 vectors over the union of their
    read lengths): every vector's exact cutoff bits, K and K' and y against
    the oracle."""
    d = dev()
    W, _ = case(m, n, seed=m + b, tag="fused")
    M = E.EffortMatrix(W, P=P, groups=G, device=d, batch=b)
    V = np.stack([synth.vector("fused", m, seed=s) for s in range(b)])
    V[1 % b] *= 7.0  # vectors of different scale in one pass
    Vt = torch.from_numpy(V).to(d)
    Y = M.matvec_batched(Vt, effort)
    torch.cuda.synchronize()
    pr = oracle.probes(W, P)
    sl = E.effort_workspace_bytes(M.desc, 1)
    ws = M.ws.cpu().numpy()
    got = M.matvec_batched_debug(Vt, effort, with_mask=m * n * b <= (1 << 26))
    for k in range(b):
        ref = oracle.run(W, pr, V[k], effort, mask=got[k]["mask"] is not None)
        # the unrecorded call's own result words and output
        res = ws[k * sl: k * sl + 16].view(np.uint32)
        assert res[0] == np.float32(ref["cutoff"]).view(np.uint32), (k, res[0])
        assert res[2] == ref["K"] and res[1] == ref["Kprime"], k
        err = rel_l2(Y[k].cpu().numpy(), ref["y"])
        assert err <= REL_L2_TOL, (k, err)
        # the recorded call (same route and kernels): the kept set
        check(got[k], ref, got[k]["mask"] is not None, where=("batched", k))
        assert rel_l2(got[k]["y"], Y[k].cpu().numpy()) < 1e-6, k
    say("fused %dx%d G=%d b=%d effort=%g ok (kept sets recorded)" % (m, n, M.groups, b, effort))
    # a second call on the same workspace gives the same result
    Y2 = M.matvec_batched(torch.from_numpy(V).to(d), effort)
    torch.cuda.synchronize()
    assert rel_l2(Y2.cpu().numpy(), Y.cpu().numpy()) < 1e-6
