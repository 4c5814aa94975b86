"""GPU parity of the Q8 bucketed format (8-byte records of 4 one-byte entries:
sign, a 4-bit level of the entry's rank bucket, 3 bits of column in an
8-column cell).  The layout is that of the quantized matrix, so the oracle
is the rule on oracle.quantize_q8(W): cutoff bits, K, K', per-row kept
counts, fingerprint, mask, y within rel-L2 1e-3 -- on the Mistral shapes,
ragged shapes, degenerate inputs, batched and multi-matrix calls and cropped
layouts.  How far the quantized product lies from the unquantized one is
printed, not asserted (it is a property of the format, not of the kernel)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from _parity import check, rel_l2  # noqa: E402

Q8 = E.EFFORT_ENTRY_Q8


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_pair(W, v, P, effort, groups=0, with_mask=True, where="", crop=0):
    d = dev()
    M = E.EffortMatrix(W, P=P, groups=groups, device=d, entry_format=Q8, crop=crop)
    assert M.desc.entry_format == Q8
    vt = torch.from_numpy(np.ascontiguousarray(v)).to(d)
    got = M.matvec_debug(vt, effort, with_mask=with_mask)
    Wq = oracle.quantize_q8(W, P)
    pr = oracle.probes(Wq, P)
    ref = (oracle.run_cropped(Wq, pr, v, effort, crop, mask=with_mask) if crop
           else oracle.run(Wq, pr, v, effort, mask=with_mask))
    err = check(got, ref, with_mask, where)
    if crop:
        assert got["crop_reached"] == ref["crop_reached"], where
    # the same kept set and tile sums; the blocks' fp32 adds into y come in
    # another order, which the "wide buckets" case (partials near 3e4 |v|
    # cancelling to a smaller y) makes visible above 1e-6
    y = M.matvec(vt, effort)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), got["y"]) < 1e-5, where
    return err


@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 14336), (14336, 4096)])
def test_q8_mistral_shapes(shape):
    m, n = shape
    W = synth.matrix("config1", m, n, seed=0)
    d = dev()
    M = E.EffortMatrix(W, P=16, device=d, entry_format=Q8)
    full, _ = E.effort_prepare_host(W, 16)
    say("q8 %dx%d: layout %.1f MB against %.1f MB (u32)" % (m, n, M.layout_bytes / 1e6,
                                                           full.total_bytes / 1e6))
    Wq = oracle.quantize_q8(W, 16)
    pr = oracle.probes(Wq, 16)
    assert np.array_equal(pr, oracle.probes(W, 16))
    for seed in range(2):
        v = synth.vector("config1", m, seed=seed)
        vt = torch.from_numpy(v).to(d)
        for effort in (1.0, 0.25, 0.125):
            with_mask = seed == 0
            got = M.matvec_debug(vt, effort, with_mask=with_mask)
            ref = oracle.run(Wq, pr, v, effort, mask=with_mask)
            err = check(got, ref, with_mask, where=(m, n, seed, effort))
            y = M.matvec(vt, effort)
            torch.cuda.synchronize()
            assert rel_l2(y.cpu().numpy(), got["y"]) < 1e-6
            unq = oracle.run(W, pr, v, effort)["y"]
            say("  q8 %dx%d seed %d effort %g ok rel-L2 %.2e; against the unquantized rule %.3f"
                % (m, n, seed, effort, err, rel_l2(got["y"], unq)))


@pytest.mark.parametrize("m,n,P,G", [(513, 2049, 16, 3), (300, 1000, 5, 0), (1000, 9000, 16, 6),
                                     (64, 8192, 8, 2), (7, 65, 3, 2), (1, 1, 1, 0), (1000, 3, 2, 0),
                                     (257, 300, 16, 5)])
@pytest.mark.parametrize("effort", [0.05, 0.3, 1.0])
def test_q8_ragged(m, n, P, G, effort):
    W = synth.weights(m, n, seed=m + n, stream=synth.stream_id("q8", "W", m, n))
    v = synth.activations(m, seed=m, stream=synth.stream_id("q8", "v", m))
    run_pair(W, v, P, effort, groups=G, where=("ragged", m, n, P, G, effort))


def test_q8_degenerate_inputs():
    W = synth.weights(64, 2000, seed=1, stream=synth.stream_id("q8deg", "W"))
    v = synth.activations(64, seed=1, stream=synth.stream_id("q8deg", "v"))
    run_pair(W, np.zeros(64, np.float32), 8, 0.25, where="zero v")  # cutoff 0: everything kept
    We = np.full((32, 960), np.float16(0.5).view(np.uint16), np.uint16)
    We[::3] |= 0x8000
    run_pair(We, np.linspace(-2, 2, 32).astype(np.float32), 4, 0.3, where="ties")
    Ws = W.copy()
    Ws[:, ::2] &= 0x83FF      # subnormals
    Ws[:, 1::7] = 0           # zeros
    Ws[:, 3::11] = 0x8000     # negative zeros
    run_pair(Ws, v, 8, 0.4, where="subnormal and signed zeros")
    run_pair(Ws, np.zeros(64, np.float32), 8, 0.4, where="signed zeros, cutoff 0")
    # sparse columns: cell steps beyond a record's header
    Wg = np.zeros((16, 4000), np.uint16)
    Wg[:, ::300] = W[:16, :14]
    run_pair(Wg, v[:16], 16, 0.5, where="steps beyond a record")
    # wide buckets: a row spanning many binades, so that level shifts are large
    Wl = W.copy()
    Wl[:, :100] = np.float16(30000.0).view(np.uint16)
    Wl[:, 100:200] = np.float16(1e-7).view(np.uint16)
    run_pair(Wl, v, 16, 0.3, where="wide buckets")
    v2 = v.copy() * 1e-3
    v2[5] = 40.0
    run_pair(W, v2, 8, 1e-7, where="K=1")


def test_q8_batched_multi_and_crop():
    d = dev()
    m, n = 1024, 4096
    W = synth.weights(m, n, seed=5, stream=synth.stream_id("q8b", "W"))
    M = E.EffortMatrix(W, P=16, device=d, batch=9, entry_format=Q8)
    Wq = oracle.quantize_q8(W, 16)
    pr = oracle.probes(Wq, 16)
    V = np.stack([synth.activations(m, seed=s, stream=synth.stream_id("q8b", "v")) for s in range(9)])
    # 9 vectors at effort 0.8: two union passes; the others: launches of up to 4
    for effort, b in ((0.25, 9), (0.8, 9), (0.25, 3), (0.1, 6)):
        got = M.matvec_batched_debug(torch.from_numpy(V[:b]).to(d), effort)
        for k in range(b):
            check(got[k], oracle.run(Wq, pr, V[k], effort), where=("batched", effort, b, k))
    W2 = synth.weights(m, 1500, seed=6, stream=synth.stream_id("q8b", "W2"))
    M2 = E.EffortMatrix(W2, P=16, device=d, entry_format=Q8)
    group = E.EffortGroup([M, M2])
    rec = E.Recorder(d)
    ys = group.matvec(torch.from_numpy(V[0]).to(d), [0.25, 0.4], record=(rec, [0, 1]))
    res = rec.results()
    for j, (Wj, e) in enumerate(((W, 0.25), (W2, 0.4))):
        Wjq = oracle.quantize_q8(Wj, 16)
        check(res[j], oracle.run(Wjq, oracle.probes(Wjq, 16), V[0], e), where=("multi", j),
              y=ys[j].cpu().numpy())
    reached = []
    for crop, effort in ((9, 0.25), (12, 0.01), (12, 0.002), (14, 0.01)):
        run_pair(W, V[1], 16, effort, crop=crop, where=("crop", crop, effort))
        reached.append(oracle.run_cropped(Wq, pr, V[1], effort, crop)["crop_reached"])
    assert any(reached) and not all(reached), reached
