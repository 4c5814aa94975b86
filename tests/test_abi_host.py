"""Host-side tests of libeffort: exported symbols, validation, and the layout.

No GPU is needed: sizing, the converter and every argument check run before
any HIP call.  The layout checks decode the prepared blob with numpy and
compare it with the input matrix and with the oracle's probes and kept sets.
"""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dynamic_sparsity_approximate_amd", "libeffort.so")
if not os.path.exists(LIB):
    subprocess.check_call([sys.executable, os.path.join(ROOT, "dynamic_sparsity_approximate_amd", "build.py")],
                          cwd=ROOT)

import dynamic_sparsity_approximate_amd as E  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from dynamic_sparsity_approximate_amd import binding as B  # noqa: E402


def rand_case(m, n, seed, tag="abi"):
    W = synth.weights(m, n, seed=seed, stream=synth.stream_id(tag, "W", m, n))
    v = synth.activations(m, seed=seed, stream=synth.stream_id(tag, "v", m))
    return W, v


def decode(desc, blob):
    m, n, P, G, TW = desc.in_dim, desc.out_dim, desc.probes_per_row, desc.groups, desc.group_width
    pr = blob[desc.off_probes: desc.off_probes + m * P * 2].view(np.uint16).reshape(m, P)
    G4 = (G + 3) // 4 * 4
    cnt = blob[desc.off_counts: desc.off_counts + m * P * G4 * 4].view(np.uint32).reshape(m, P, G4)[:, :, :G]
    ent = blob[desc.off_entries: desc.off_entries + m * desc.row_stride * 4].view(np.uint32)
    return pr, cnt, ent.reshape(m, desc.row_stride)


def decode_rowmax(desc, blob):
    return blob[desc.off_rowmax: desc.off_rowmax + desc.in_dim * 2].view(np.uint16)


# ---------------------------------------------------------------- symbols

def test_library_exports_every_declared_function():
    names = B.header_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(LIB)
    for name in names:
        assert hasattr(lib, name), name


def test_strerror_names_codes():
    assert E.effort_strerror(0) == "ok"
    assert "invalid" in E.effort_strerror(1)
    assert E.effort_strerror(99) == "unknown status"


# ---------------------------------------------------------------- sizing

def test_layout_bytes_and_groups():
    assert E.effort_default_groups(14336) == 4
    assert E.effort_default_groups(4096) == 2
    assert E.effort_default_groups(1024) == 2
    assert E.effort_default_groups(12288) == 4  # powers of two only
    assert E.effort_default_groups(32000) == 8
    m, n, P = 4096, 14336, 16
    nb = E.effort_layout_bytes(m, n, P)
    # entries dominate: 4 bytes per weight, plus probes and counts (4 groups)
    assert nb >= 4 * m * n + 2 * m * P + 4 * m * P * 4 + 2 * m
    assert nb < 4 * m * n + 2 * m * P + 4 * m * P * 4 + 2 * m + 5 * 256


@pytest.mark.parametrize("args,code", [
    ((0, 10, 1, 0), B.EFFORT_EINVAL), ((10, 0, 1, 0), B.EFFORT_EINVAL),
    ((10, 10, 0, 0), B.EFFORT_EINVAL), ((10, 10, 11, 0), B.EFFORT_EINVAL),
    ((10, 10, 1, -1), B.EFFORT_EINVAL), ((10, 100000, 1, 1), B.EFFORT_EUNSUPPORTED),
    ((2**31, 8, 1, 0), B.EFFORT_EUNSUPPORTED),
])
def test_layout_bytes_rejects(args, code):
    with pytest.raises(E.EffortError) as ei:
        E.effort_layout_bytes_ex(*args)
    assert ei.value.code == code


def test_group_geometry_covers_columns():
    for n, g in [(100, 8), (1000, 3), (14336, 8), (641, 2), (64, 64), (8192, 1)]:
        W, _ = rand_case(2, n, seed=1)
        d, _ = E.effort_prepare_host(W, 1, g)
        assert d.group_width % 64 == 0
        assert (d.groups - 1) * d.group_width < n <= d.groups * d.group_width
        assert d.row_stride == d.groups * d.group_width


# ---------------------------------------------------------------- converter

@pytest.mark.parametrize("m,n,P,G", [(5, 37, 3, 0), (9, 300, 16, 3), (4, 64, 64, 1), (3, 130, 7, 3),
                                     (16, 256, 16, 0), (1, 1, 1, 0)])
def test_layout_roundtrip_and_order(m, n, P, G):
    W, _ = rand_case(m, n, seed=m + n + P)
    if m > 2:
        W[1, ::3] = W[1, 0]  # ties
        W[2, : n // 2] = 0   # zeros
    d, blob = E.effort_prepare_host(W, P, G)
    E.effort_layout_check(d, blob)
    pr, cnt, ent = decode(d, blob)
    TW = d.group_width
    assert np.array_equal(decode_rowmax(d, blob), (W & 0x7FFF).max(axis=1))
    # probes are the oracle's order statistics
    ref = oracle.probes(W, P)
    assert np.array_equal(pr.view(np.float16).astype(np.float32), ref)
    for i in range(m):
        # whole-row rank of each column: |w| descending, column ascending
        keys = (W[i] & 0x7FFF).astype(np.int64)
        order = np.lexsort((np.arange(n), -keys))
        rank = np.empty(n, np.int64)
        rank[order] = np.arange(1, n + 1)
        seen = np.zeros(n, bool)
        for g in range(d.groups):
            width = min(TW, n - g * TW)
            run = ent[i, g * TW: g * TW + width]
            vals = (run & 0xFFFF).astype(np.uint16)
            cols = g * TW + (run >> 16).astype(np.int64)
            assert np.all((run >> 16) < width)
            assert np.array_equal(vals, W[i, cols])         # values round-trip
            assert not seen[cols].any()
            seen[cols] = True
            assert np.all(np.diff(rank[cols]) > 0)          # rank order inside the group
            for k in range(P):
                Rk = -(-(k + 1) * n // P)
                assert cnt[i, k, g] == np.sum(rank[cols] <= Rk)
            assert np.all(ent[i, g * TW + width: (g + 1) * TW] == 0)  # padding
        assert seen.all()


def test_converter_rejects_nonfinite_and_small_buffer():
    W, _ = rand_case(4, 8, seed=2)
    W[1, 3] = 0x7C00  # +inf
    with pytest.raises(E.EffortError) as ei:
        E.effort_prepare_host(W, 2)
    assert ei.value.code == B.EFFORT_EINVAL
    W[1, 3] = 0xFE00  # NaN
    with pytest.raises(E.EffortError):
        E.effort_prepare_host(W, 2)
    W[1, 3] = 0
    d = E.effort_desc()
    small = np.zeros(64, np.uint64)
    rc = B.lib().effort_prepare_host(W.ctypes.data, 4, 8, 2, small.ctypes.data, 512, ctypes.byref(d))
    assert rc == B.EFFORT_ENOSPACE


def test_layout_check_detects_corruption():
    W, _ = rand_case(8, 40, seed=3)
    d, blob = E.effort_prepare_host(W, 4)
    bad = blob.copy()
    bad[d.off_entries + 17] ^= 1
    with pytest.raises(E.EffortError) as ei:
        E.effort_layout_check(d, bad)
    assert ei.value.code == B.EFFORT_ECORRUPT
    d2 = d.copy()
    d2.magic ^= 1
    with pytest.raises(E.EffortError) as ei:
        E.effort_layout_check(d2, blob)
    assert ei.value.code == B.EFFORT_ECORRUPT
    d3 = d.copy()
    d3.out_dim += 1  # descriptor check fails
    with pytest.raises(E.EffortError) as ei:
        E.effort_layout_check(d3, blob)
    assert ei.value.code == B.EFFORT_ECORRUPT


# ---------------------------------------------------------------- layout walk against the oracle

def _threshold(av, cutoff):
    """Smallest fp16 magnitude key k with fl32(av * k) >= cutoff (0x7C00: none), by bisection."""
    keys = np.arange(0x7C00, dtype=np.uint16)
    mags = keys.view(np.float16).astype(np.float32)
    ok = (np.float32(av) * mags) >= np.float32(cutoff)
    idx = np.nonzero(ok)[0]
    return int(idx[0]) if idx.size else 0x7C00


@pytest.mark.parametrize("m,n,P,G,effort", [(64, 300, 16, 3, 0.25), (32, 128, 4, 2, 0.6),
                                            (48, 200, 200, 1, 0.1), (20, 70, 1, 2, 0.5)])
def test_run_prefix_contains_exactly_the_kept_entries(m, n, P, G, effort):
    """The (row, group) read length the multiply uses covers every kept entry,
    and the keep test on the key equals the oracle's product test."""
    W, v = rand_case(m, n, seed=P)
    d, blob = E.effort_prepare_host(W, P, G)
    pr, cnt, ent = decode(d, blob)
    ref = oracle.run(W, oracle.probes(W, P), v, effort, mask=True)
    TW = d.group_width
    for i in range(m):
        t = _threshold(abs(v[i]), ref["cutoff"])
        q = int(np.sum(pr[i] >= t))
        assert q == ref["row_chart_kept"][i]
        for g in range(d.groups):
            width = min(TW, n - g * TW)
            L = int(cnt[i, min(q, P - 1), g])
            run = ent[i, g * TW: g * TW + width]
            keep = (run & 0x7FFF) >= t
            cols = g * TW + (run >> 16).astype(np.int64)
            assert np.array_equal(keep, ref["mask"][i, cols].astype(bool))
            assert not keep[L:].any()
            # kept entries form a prefix of the run
            assert np.all(keep[: keep.sum()])


# ---------------------------------------------------------------- matvec validation (no HIP call is reached)

def _desc_and_blob():
    W, _ = rand_case(16, 64, seed=4)
    return E.effort_prepare_host(W, 4)


FAKE = 1 << 40  # 256-aligned fake device address: never dereferenced, validation fails first


@pytest.mark.parametrize("effort", [0.0, -1.0, 1.5, float("nan"), float("inf")])
def test_matvec_rejects_effort(effort):
    d, _ = _desc_and_blob()
    ws = E.effort_workspace_bytes(d, 1)
    with pytest.raises(E.EffortError) as ei:
        E.effort_matvec(d, FAKE, FAKE, effort, FAKE, FAKE, ws)
    assert ei.value.code == B.EFFORT_EINVAL


def test_matvec_rejects_bad_buffers_and_descriptors():
    d, _ = _desc_and_blob()
    ws = E.effort_workspace_bytes(d, 1)
    cases = [
        (dict(layout=None), B.EFFORT_EINVAL),
        (dict(v=None), B.EFFORT_EINVAL),
        (dict(y=None), B.EFFORT_EINVAL),
        (dict(ws=None), B.EFFORT_EINVAL),
        (dict(layout=FAKE + 16), B.EFFORT_EINVAL),
        (dict(ws=FAKE + 8), B.EFFORT_EINVAL),
        (dict(v=FAKE + 2), B.EFFORT_EINVAL),
        (dict(ws_bytes=ws - 1), B.EFFORT_ENOSPACE),
    ]
    for over, code in cases:
        a = dict(layout=FAKE, v=FAKE, y=FAKE, ws=FAKE, ws_bytes=ws)
        a.update(over)
        with pytest.raises(E.EffortError) as ei:
            E.effort_matvec(d, a["layout"], a["v"], 0.25, a["y"], a["ws"], a["ws_bytes"])
        assert ei.value.code == code, over
    for field in ("magic", "version", "groups", "desc_check", "off_entries"):
        d2 = d.copy()
        setattr(d2, field, getattr(d2, field) + 1)
        with pytest.raises(E.EffortError) as ei:
            E.effort_matvec(d2, FAKE, FAKE, 0.25, FAKE, FAKE, ws)
        assert ei.value.code == B.EFFORT_ECORRUPT, field
    for batch in (0, 17):
        with pytest.raises(E.EffortError) as ei:
            E.effort_matvec_batched(d, FAKE, FAKE, batch, 0.25, FAKE, FAKE, ws * 17)
        assert ei.value.code == B.EFFORT_EINVAL
    # b slices, then the union read lengths [G][m] and their per-256-row sums
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    m, G = int(d.in_dim), int(d.groups)
    wb4 = 4 * ws + up(G * m * 4) + up(-(-m // 256) * (G + 1) * 4)
    assert E.effort_workspace_bytes(d, 4) == wb4
    with pytest.raises(E.EffortError) as ei:
        E.effort_matvec_batched(d, FAKE, FAKE, 4, 0.25, FAKE, FAKE, wb4 - 1)
    assert ei.value.code == B.EFFORT_ENOSPACE
    with pytest.raises(E.EffortError):
        E.effort_workspace_bytes(d, 0)


def test_dense_and_glue_validation():
    for args in [(None, FAKE, 4, 4, FAKE), (FAKE, FAKE, 0, 4, FAKE), (FAKE, FAKE, 4, 0, FAKE),
                 (FAKE + 1, FAKE, 4, 4, FAKE)]:
        with pytest.raises(E.EffortError) as ei:
            E.dense_gemv(*args)
        assert ei.value.code == B.EFFORT_EINVAL
    with pytest.raises(E.EffortError):
        E.dense_gemm_small(FAKE, FAKE, 17, 4, 4, FAKE)
    with pytest.raises(E.EffortError):
        E.effort_silu_mul(FAKE, FAKE, 0, FAKE)
    for args in [(None, 1.0, FAKE, 1.0, 4, FAKE), (FAKE, 1.0, FAKE, 1.0, 0, FAKE),
                 (FAKE + 2, 1.0, FAKE, 1.0, 4, FAKE)]:
        with pytest.raises(E.EffortError) as ei:
            E.effort_axpby(*args)
        assert ei.value.code == B.EFFORT_EINVAL


def test_multi_sizes_and_rejects():
    descs = [E.effort_prepare_host(rand_case(16, n, seed=10 + n)[0], 4)[0] for n in (64, 128, 96)]
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    single = [E.effort_workspace_bytes(d, 1) for d in descs]
    assert E.effort_workspace_bytes_multi(descs) == sum(up(b) for b in single)
    assert E.effort_workspace_bytes_multi(descs[:1]) == up(single[0])
    ws = E.effort_workspace_bytes_multi(descs)
    good = dict(descs=descs, layouts=[FAKE] * 3, vs=[FAKE] * 3, efforts=[0.25] * 3, ys=[FAKE] * 3,
                ws=FAKE, ws_bytes=ws)
    cases = [
        (dict(descs=descs + descs[:2], layouts=[FAKE] * 5, vs=[FAKE] * 5, efforts=[0.25] * 5,
              ys=[FAKE] * 5), B.EFFORT_EINVAL),  # more than EFFORT_MAX_MULTI
        (dict(vs=[FAKE, None, FAKE]), B.EFFORT_EINVAL),
        (dict(vs=[FAKE, FAKE + 2, FAKE]), B.EFFORT_EINVAL),
        (dict(efforts=[0.25, 0.0, 0.25]), B.EFFORT_EINVAL),
        (dict(efforts=[0.25, 0.25, float("nan")]), B.EFFORT_EINVAL),
        (dict(layouts=[FAKE, None, FAKE]), B.EFFORT_EINVAL),
        (dict(layouts=[FAKE, FAKE + 16, FAKE]), B.EFFORT_EINVAL),
        (dict(ys=[FAKE, FAKE, FAKE + 2]), B.EFFORT_EINVAL),
        (dict(ws=FAKE + 8), B.EFFORT_EINVAL),
        (dict(ws_bytes=ws - 1), B.EFFORT_ENOSPACE),
    ]
    for over, code in cases:
        a = dict(good)
        a.update(over)
        with pytest.raises(E.EffortError) as ei:
            E.effort_matvec_multi(a["descs"], a["layouts"], a["vs"], a["efforts"], a["ys"], a["ws"],
                                  a["ws_bytes"])
        assert ei.value.code == code, over
    with pytest.raises(E.EffortError) as ei:
        E.effort_workspace_bytes_multi([])
    assert ei.value.code == B.EFFORT_EINVAL


# ---------------------------------------------------------------- error handling of the binding

def test_binding_reinitialises_workspace_after_hip_error(monkeypatch):
    """A call that fails with EFFORT_EHIP part-way may leave set the workspace
    words every call expects to find zero; the binding zero-fills the
    workspace again before raising.  The library is replaced by a stand-in
    that reports the error, so nothing runs on a device."""
    calls = []
    real = B._lib

    class StandIn:
        def __getattr__(self, name):
            return getattr(real, name)

        def _fail(self, name, code):
            def f(*args):
                calls.append((name,))
                return code
            return f

        def effort_workspace_init(self, ws, nbytes, stream):
            calls.append(("init", ws, nbytes))
            return B.EFFORT_OK

    fake = StandIn()
    monkeypatch.setattr(B, "_lib", fake)
    desc, blob = _desc_and_blob()
    ws = np.zeros(4096, np.uint8)  # host memory standing in for a device workspace
    v = np.zeros(desc.in_dim, np.float32)
    y = np.zeros(desc.out_dim, np.float32)
    entries = [
        ("effort_matvec", lambda: B.effort_matvec(desc, blob, v, 0.25, y, ws, ws.size)),
        ("effort_matvec_batched", lambda: B.effort_matvec_batched(desc, blob, v, 1, 0.25, y, ws, ws.size)),
        ("effort_matvec_debug", lambda: B.effort_matvec_debug(desc, blob, v, 0.25, y, ws, ws.size)),
        ("effort_matvec_batched_debug",
         lambda: B.effort_matvec_batched_debug(desc, blob, v, 1, 0.25, y, ws, ws.size)),
        ("effort_matvec_multi", lambda: B.effort_matvec_multi([desc], [blob], v, 0.25, [y], ws, ws.size)),
        ("effort_matvec_multi_debug",
         lambda: B.effort_matvec_multi_debug([desc], [blob], v, 0.25, [y], ws, ws.size)),
    ]
    for name, call in entries:
        for code in (B.EFFORT_EHIP, B.EFFORT_EINVAL):
            calls.clear()
            monkeypatch.setattr(StandIn, name, lambda self, *a, _n=name, _c=code: (calls.append((_n,)), _c)[1],
                                raising=False)
            with pytest.raises(E.EffortError) as ei:
                call()
            assert ei.value.code == code, name
            if code == B.EFFORT_EHIP:
                assert calls == [(name,), ("init", ws.ctypes.data, ws.size)], (name, calls)
            else:
                assert calls == [(name,)], (name, calls)


# ---------------------------------------------------------------- layout options: crop, r12 / q8 records

def q8_level(lo, hi, code):
    """Level `code` of the Q8 bucket [lo, hi]: lo + code 2^s capped at hi, s the
    smallest shift with 15 2^s >= hi - lo."""
    s = 0
    while (15 << s) < hi - lo:
        s += 1
    return min(lo + (code << s), hi)


def decode_runs(desc, blob):
    """Per (row, group): the storage units of the run decoded to a list of
    (unit index, in-group column, value bits[, q8: header segment]) in storage
    order; unused record slots are dropped.  Also the counts table [m][P][G]."""
    m, P, G = desc.in_dim, desc.probes_per_row, desc.groups
    G4 = (G + 3) // 4 * 4
    cnt = blob[desc.off_counts: desc.off_counts + m * P * G4 * 4].view(np.uint32).reshape(m, P, G4)[:, :, :G]
    uw = {B.EFFORT_ENTRY_U32: 1, B.EFFORT_ENTRY_R12: 3, B.EFFORT_ENTRY_Q8: 2}[desc.entry_format]
    probes = blob[desc.off_probes: desc.off_probes + m * P * 2].view(np.uint16).reshape(m, P)
    rowmax = decode_rowmax(desc, blob)
    words = blob[desc.off_entries: desc.off_entries + m * desc.row_stride * uw * 4].view(np.uint32)
    words = words.reshape(m, G, desc.group_stride * uw)
    runs = {}
    for i in range(m):
        for g in range(G):
            L = int(cnt[i, P - 1, g])
            w = words[i, g]
            out = []
            if uw == 1:
                for u in range(L):
                    out.append((u, int(w[u] >> 16), int(w[u] & 0xFFFF)))
            elif uw == 2:
                for u in range(L):
                    h, e = int(w[2 * u]), int(w[2 * u + 1])
                    seg, last, cell = h & 15, (h >> 4) & 3, (h >> 6) & 511
                    steps = ((h >> 15) & 63, (h >> 21) & 63, h >> 27)
                    lo = int(probes[i, seg])
                    hi = int(rowmax[i]) if seg == 0 else int(probes[i, seg - 1])
                    for t in range(last + 1):
                        if t:
                            cell += steps[t - 1]
                        b = (e >> (8 * t)) & 255
                        key = q8_level(lo, hi, (b >> 3) & 15)
                        out.append((u, cell * 8 + (b & 7), key | ((b >> 7) << 15), seg))
            else:
                for u in range(L):
                    w0, w1, w2 = (int(x) for x in w[3 * u: 3 * u + 3])
                    vals = [w0 & 0xFFFF, w0 >> 16, w1 & 0xFFFF, w1 >> 16]
                    c0 = w2 & 0xFFF
                    c1 = c0 + ((w2 >> 12) & 0x7F)
                    c2 = c1 + ((w2 >> 19) & 0x7F)
                    c3 = c2 + (w2 >> 26)
                    for c, val in zip((c0, c1, c2, c3), vals):
                        if val != 0x8000:
                            out.append((u, c, val))
            runs[(i, g)] = out
    return cnt, runs


@pytest.mark.parametrize("m,n,P,G,fmt,crop", [
    (9, 300, 16, 3, 0, 12), (6, 1000, 16, 2, 1, 0), (6, 1000, 16, 2, 1, 9), (5, 37, 3, 0, 1, 0),
    (4, 4096, 16, 1, 1, 16), (3, 130, 7, 3, 0, 1), (8, 5000, 8, 0, 1, 5), (2, 64, 64, 1, 1, 40),
    (9, 300, 16, 3, 2, 12), (6, 1000, 16, 2, 2, 0), (5, 37, 3, 0, 2, 0), (4, 4096, 16, 1, 2, 16),
    (8, 5000, 8, 0, 2, 5), (7, 700, 16, 2, 2, 3), (3, 20, 1, 1, 2, 0)])
def test_layout_options_roundtrip(m, n, P, G, fmt, crop):
    """Every stored pair exactly once, in its segment, in the format's order;
    probes, rowmax and floor.  A q8 layout is the layout of the quantized
    matrix (oracle.quantize_q8): its values, ranks, crop and floor."""
    W, _ = rand_case(m, n, seed=m + n + P + crop, tag="opts")
    if m > 2:
        W[1, ::3] = W[1, 0]        # ties
        W[2, : n // 2] = 0         # zeros
        W[2, n // 2: n // 2 + 5] = 0x8000  # negative zeros
    d, blob = E.effort_prepare_host(W, P, G, fmt, crop)
    if fmt == B.EFFORT_ENTRY_Q8:
        Wq = oracle.quantize_q8(W, P)
        assert np.array_equal(oracle.probes(Wq, P), oracle.probes(W, P))
        W = Wq
    E.effort_layout_check(d, blob)
    assert d.total_bytes == E.effort_layout_bytes_opts(W, P, G, fmt, crop) <= blob.size
    c = crop or P
    assert d.entry_format == fmt and d.crop_segments == c
    assert d.index_bytes == (2 if fmt == 0 else 0)
    st = oracle.stored_mask(W, P, c)
    pr, _, _ = decode(d, blob) if fmt == 0 else (None, None, None)
    probes = blob[d.off_probes: d.off_probes + m * P * 2].view(np.uint16).reshape(m, P)
    assert np.array_equal(probes.view(np.float16).astype(np.float32), oracle.probes(W, P))
    assert np.array_equal(decode_rowmax(d, blob), (W & 0x7FFF).max(axis=1))
    if c < P:
        floor = blob[d.off_floor: d.off_floor + m * 2].view(np.uint16)
        for i in range(m):
            dropped = (W[i] & 0x7FFF)[st[i] == 0]
            assert floor[i] == (dropped.max() if dropped.size else 0)
    else:
        assert d.off_floor == 0
    cnt, runs = decode_runs(d, blob)
    TW = d.group_width
    for i in range(m):
        keys = (W[i] & 0x7FFF).astype(np.int64)
        order = np.lexsort((np.arange(n), -keys))
        rank = np.empty(n, np.int64)
        rank[order] = np.arange(1, n + 1)
        seg = np.searchsorted([-(-(k + 1) * n // P) for k in range(P)], rank)  # segment of each column
        seen = np.zeros(n, bool)
        for g in range(d.groups):
            width = min(TW, n - g * TW)
            ents = runs[(i, g)]
            assert int(cnt[i, P - 1, g]) <= d.group_stride
            for k in range(c, P):  # constant past the crop
                assert cnt[i, k, g] == cnt[i, c - 1, g]
            cols = np.array([g * TW + e[1] for e in ents], np.int64)
            vals = np.array([e[2] for e in ents], np.int64)
            units = np.array([e[0] for e in ents], np.int64)
            assert np.all(cols - g * TW < width)
            want_vals = W[i, cols].astype(np.int64)
            if fmt == 1:
                want_vals[want_vals == 0x8000] = 0  # -0 stored as +0
            assert np.array_equal(vals, want_vals)
            assert not seen[cols].any()
            seen[cols] = True
            # every unit lies in the segment the counts table gives it
            lo = np.concatenate([[0], cnt[i, :, g][:-1]]).astype(np.int64)
            for k in range(c):
                inside = (units >= lo[k]) & (units < cnt[i, k, g])
                assert np.all(seg[cols[inside]] == k), (i, g, k)
                if fmt == B.EFFORT_ENTRY_Q8:
                    assert all(e[3] == k for e, x in zip(ents, inside) if x)
                ck = cols[inside]
                if fmt == 0:
                    assert np.all(np.diff(rank[ck]) > 0)  # rank order in the segment
                else:
                    assert np.all(np.diff(ck) > 0)        # column order in the segment
        assert np.array_equal(seen, st[i].astype(bool))  # exactly the stored pairs


def test_r12_records_are_three_bytes_per_entry():
    """At 4096 columns and P = 16 (a step above 63 or 127 columns is rare) the
    records hold close to 4 entries: the entries region is within a few
    percent of 3 bytes per weight, against 4 for the u32 format."""
    W, _ = rand_case(64, 4096, seed=7, tag="r12size")
    d, blob = E.effort_prepare_host(W, 16, 1, B.EFFORT_ENTRY_R12)
    ent_bytes = d.off_rowmax - d.off_entries
    assert ent_bytes <= 3.1 * W.size
    cnt, runs = decode_runs(d, blob)
    used = sum(int(cnt[i, 15, 0]) for i in range(64))
    assert used * 4 <= 1.03 * W.size  # record slots per weight


def test_q8_records_are_two_bytes_per_entry():
    """Q8 at 4096 columns and P = 16: 8-byte records of close to 4 entries."""
    W, _ = rand_case(64, 4096, seed=7, tag="q8size")
    d, blob = E.effort_prepare_host(W, 16, 1, B.EFFORT_ENTRY_Q8)
    assert d.off_rowmax - d.off_entries <= 2.1 * W.size
    cnt, runs = decode_runs(d, blob)
    used = sum(int(cnt[i, 15, 0]) for i in range(64))
    assert used * 4 <= 1.03 * W.size


def test_layout_options_reject():
    W, _ = rand_case(4, 9000, seed=8, tag="rej")
    for fmt in (B.EFFORT_ENTRY_R12, B.EFFORT_ENTRY_Q8):  # 12-bit columns, 9-bit cells
        with pytest.raises(E.EffortError) as ei:
            E.effort_prepare_host(W, 16, 1, fmt)
        assert ei.value.code == B.EFFORT_EUNSUPPORTED
    with pytest.raises(E.EffortError) as ei:  # a 4-bit segment field
        E.effort_prepare_host(W[:, :4096], 17, 1, B.EFFORT_ENTRY_Q8)
    assert ei.value.code == B.EFFORT_EUNSUPPORTED
    for bad in ((3, 0), (0, 17), (0, -1)):
        with pytest.raises(E.EffortError) as ei:
            E.effort_prepare_host(W, 16, 0, *bad)
        assert ei.value.code == B.EFFORT_EINVAL
