"""The allocation-free entry point (effort_matvec_noalloc): the same kernels as
effort_matvec with the workspace in the library's static device array.  Its
output is compared with effort_matvec's on the same inputs (the same cutoff and
kept set; only the order of the fp32 atomics of the flush differs, so rel-L2
<= 1e-5 is asked) and with the oracle (rel-L2 1e-3), on calls in a row whose
second input is smaller than the first, in the three entry formats (the
oracle of a q8 layout runs on the quantized matrix), and the size limit is
checked on the host."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from _parity import rel_l2  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.gpu
def test_noalloc_matches_matvec_on_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda:0")
    U32, R12, Q8 = E.EFFORT_ENTRY_U32, E.EFFORT_ENTRY_R12, E.EFFORT_ENTRY_Q8
    cases = [(4096, 14336, 0.25, 0, R12), (513, 2049, 0.3, 1, U32), (4096, 14336, 0.125, 2, U32),
             (300, 1000, 1.0, 3, Q8), (1000, 3000, 0.2, 4, R12)]
    for m, n, effort, seed, fmt in cases:
        W = synth.weights(m, n, seed=seed, stream=synth.stream_id("noalloc", "W", m, n))
        v = synth.activations(m, seed=seed, stream=synth.stream_id("noalloc", "v", m))
        M = E.EffortMatrix(W, P=16, device=d, entry_format=fmt)
        vt = torch.from_numpy(v).to(d)
        y_ref = M.matvec(vt, effort)
        y = torch.full((n,), float("nan"), dtype=torch.float32, device=d)
        E.effort_matvec_noalloc(M.desc, M.layout, vt, effort, y)
        torch.cuda.synchronize()
        y, y_ref = y.cpu().numpy(), y_ref.cpu().numpy()
        assert rel_l2(y, y_ref) <= 1e-5, (m, n, rel_l2(y, y_ref))
        Wr = oracle.quantize_q8(W, 16) if fmt == Q8 else W
        ref = oracle.run(Wr, oracle.probes(Wr, 16), v, effort)
        err = rel_l2(y, ref["y"])
        assert err <= 1e-3, (m, n, fmt, err)
        say("noalloc %dx%d effort %g format %d: rel-L2 %.2e against effort_matvec, %.2e against the oracle" % (
            m, n, effort, fmt, rel_l2(y, y_ref), err))


def test_noalloc_rejects_matrices_beyond_its_workspace():
    """Checked on the host before any device work: a matrix whose workspace
    exceeds the static array is ENOSPACE (no GPU needed)."""
    m, n, P = 140000, 64, 16  # candidate list alone: 140000 * 16 * 4 bytes > 8 MiB
    W = synth.weights(m, n, seed=0, stream=1)
    desc, _ = E.effort_prepare_host(W, P)
    assert E.effort_workspace_bytes(desc, 1) > E.EFFORT_NOALLOC_WORKSPACE_BYTES
    with pytest.raises(E.EffortError) as ei:
        E.effort_matvec_noalloc(desc, 256, 256, 0.25, 256)
    assert ei.value.code == E.EFFORT_ENOSPACE
