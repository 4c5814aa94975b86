"""Pins of the oracle against things other than itself.

Each test ties one oracle function to a library routine (numpy's float16
conversion, sort, float64 matmul), a closed form, a hand-worked case, brute
force over tiny inputs or a theorem of the rule (nesting, scaling, dropped-mass
bound, kept-fraction bound).  A dropped term, a wrong sign or index, or a
transposed operand in oracle.c fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def mags(W):
    return np.abs(W.view(np.float16).astype(np.float64))


def vals(W):
    return W.view(np.float16).astype(np.float64)


def fl32_prod(a, b):
    # product of two fp32-representable numbers is exact in double; one rounding to fp32
    return (np.asarray(a, dtype=np.float64) * np.asarray(b, dtype=np.float64)).astype(np.float32)


def expected_K(effort, N):
    k = math.ceil(Fraction(float(np.float32(effort))) * N)
    return min(N, max(1, k))


def rand_case(m, n, seed, tag="pin"):
    W = synth.weights(m, n, seed=seed, stream=synth.stream_id(tag, "W", m, n))
    v = synth.activations(m, seed=seed, stream=synth.stream_id(tag, "v", m))
    return W, v


# ---------------------------------------------------------------- primitives

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


def test_pair_hash_is_splitmix64():
    # first output of splitmix64 seeded with 0 (Vigna's reference implementation)
    assert oracle.pair_hash(0) == 0xE220A8397B1DCDAF
    for x in [1, 2, 12345, 2**40 + 17, 2**64 - 1]:
        assert oracle.pair_hash(x) == synth.splitmix64(x)


def test_probes_are_order_statistics():
    for (m, n, P) in [(5, 37, 1), (5, 37, 3), (7, 64, 16), (3, 100, 7), (4, 9, 9)]:
        W, _ = rand_case(m, n, seed=m * n + P)
        got = oracle.probes(W, P)
        srt = -np.sort(-mags(W), axis=1)
        for k in range(P):
            rank = -(-(k + 1) * n // P)
            assert np.array_equal(got[:, k].astype(np.float64), srt[:, rank - 1])
        # probes descend along a row and the last one is the row minimum
        assert np.all(np.diff(got, axis=1) <= 0)
        assert np.array_equal(got[:, -1].astype(np.float64), mags(W).min(axis=1))


def test_probes_with_P_equal_n_list_every_magnitude():
    W, _ = rand_case(6, 20, seed=3)
    got = oracle.probes(W, 20).astype(np.float64)
    assert np.array_equal(got, -np.sort(-mags(W), axis=1))


def test_chart_is_exact_fp32_product():
    W, v = rand_case(64, 48, seed=5)
    pr = oracle.probes(W, 8)
    v = v.copy()
    v[::7] *= -1
    v[3] = 0.0
    got = oracle.chart(v, pr)
    ref = fl32_prod(np.abs(v)[:, None], pr)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- cutoff

@pytest.mark.parametrize("seed", range(6))
def test_cutoff_is_kth_largest(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 3000))
    ch = rng.choice(rng.random(max(1, N // 4)).astype(np.float32), size=N)  # many ties
    ch[rng.random(N) < 0.1] = 0.0
    for effort in [1e-6, 0.01, 0.12, 0.16, 0.25, 0.5, 0.999, 1.0]:
        K, c, Kp = oracle.cutoff(ch, effort)
        assert K == expected_K(effort, N)
        assert c == np.sort(ch)[::-1][K - 1]
        assert c in ch
        assert np.sum(ch > c) < K <= np.sum(ch >= c) == Kp


def test_K_examples():
    # K = ceil(effort * N) with effort taken as its fp32 value
    assert expected_K(0.16, 65536) == 10486
    assert expected_K(0.12, 229376) == 27526
    ch = np.arange(65536, dtype=np.float32)
    assert oracle.cutoff(ch, 0.16)[0] == 10486
    assert oracle.cutoff(np.ones(229376, np.float32), 0.12)[0] == 27526
    assert oracle.cutoff(np.ones(10, np.float32), 1e-30)[0] == 1


@pytest.mark.parametrize("effort", [0.0, -0.25, 1.0000001, float("nan"), float("inf")])
def test_cutoff_rejects_effort_outside_unit_interval(effort):
    with pytest.raises(ValueError):
        oracle.cutoff(np.ones(4, np.float32), effort)


def test_invalid_shapes_rejected():
    W, v = rand_case(4, 8, seed=1)
    with pytest.raises(ValueError):
        oracle.probes(W, 9)
    with pytest.raises(ValueError):
        oracle.probes(W, 0)
    with pytest.raises(ValueError):
        oracle.probes(np.zeros((0, 8), np.uint16), 1)


# ---------------------------------------------------------------- hand-worked case

def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    W = np.array(g["W"], dtype=np.float16).view(np.uint16)
    v = np.array(g["v"], dtype=np.float32)
    pr = oracle.probes(W, g["P"])
    assert pr.tolist() == g["probes"]
    assert oracle.chart(v, pr).tolist() == g["chart"]
    for case in g["cases"]:
        r = oracle.run(W, pr, v, case["effort"], mask=True)
        assert r["K"] == case["K"] and r["Kprime"] == case["Kprime"]
        assert float(r["cutoff"]) == case["cutoff"]
        assert r["mask"].tolist() == case["mask"]
        assert r["y"].tolist() == case["y"]


# ---------------------------------------------------------------- I1: effort = 1 is dense

@pytest.mark.parametrize("shape,P", [((256, 256), 16), ((37, 101), 5), ((1, 1), 1), ((300, 17), 17)])
def test_effort_one_is_dense(shape, P):
    W, v = rand_case(*shape, seed=11)
    pr = oracle.probes(W, P)
    r = oracle.run(W, pr, v, 1.0, mask=True)
    assert r["mask"].all()
    assert r["total_kept"] == W.size
    yd = oracle.dense(W, v)
    assert np.array_equal(r["y"], yd)  # same double order
    ref = v.astype(np.float64) @ vals(W)
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- BF: brute force on tiny inputs

def _bf_case(W, v, P, effort):
    """Chart entries enumerated directly from sorted magnitudes, kept set by enumeration."""
    m, n = W.shape
    mg = mags(W)
    av = np.abs(v.astype(np.float64))
    chart = []
    for i in range(m):
        s = sorted(mg[i], reverse=True)
        for k in range(P):
            rank = -(-(k + 1) * n // P)
            chart.append(float(fl32_prod(av[i], s[rank - 1])))
    N = len(chart)
    K = expected_K(effort, N)
    cut = sorted(chart, reverse=True)[K - 1]
    kept = np.zeros((m, n), np.uint8)
    for i in range(m):
        for j in range(n):
            kept[i, j] = float(fl32_prod(av[i], mg[i, j])) >= cut
    y = np.zeros(n)
    for i in range(m):
        for j in range(n):
            if kept[i, j]:
                y[j] += float(v[i]) * vals(W)[i, j]
    return K, cut, kept, y


@pytest.mark.parametrize("seed", range(8))
def test_bruteforce_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    m, n = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    W, v = rand_case(m, n, seed=seed, tag="bf")
    if seed % 2:  # ties and zeros
        W = W.copy()
        W[rng.random(W.shape) < 0.3] = W.flat[0]
        W[rng.random(W.shape) < 0.1] = 0
    for P in sorted({1, min(2, n), n}):
        pr = oracle.probes(W, P)
        N = m * P
        for K in range(1, N + 1):
            effort = np.float32(K / N)
            r = oracle.run(W, pr, v, float(effort), mask=True)
            Kb, cut, kept, y = _bf_case(W, v, P, float(effort))
            assert r["K"] == Kb
            assert float(r["cutoff"]) == cut
            assert np.array_equal(r["mask"], kept)
            assert np.allclose(r["y"], y, rtol=1e-15, atol=1e-300)


def test_P_equal_n_selects_top_products():
    # With P = n the chart is every product, so the kept set is the K largest
    # products (plus those tied with the K-th).
    W, v = rand_case(6, 7, seed=42)
    pr = oracle.probes(W, 7)
    prod = fl32_prod(np.abs(v)[:, None], mags(W)).astype(np.float64)
    order = np.sort(prod.ravel())[::-1]
    for K0 in [1, 5, 13, 42]:
        effort = float(np.float32(K0 / 42))
        K = expected_K(effort, 42)
        r = oracle.run(W, pr, v, effort, mask=True)
        assert r["K"] == K and K in (K0, K0 + 1)
        assert r["total_kept"] == np.sum(prod >= order[K - 1])
        assert np.array_equal(r["mask"].astype(bool), prod >= order[K - 1])


# ---------------------------------------------------------------- I3: kept-fraction bound

@pytest.mark.parametrize("shape,P", [((256, 256), 16), ((256, 256), 1), ((256, 256), 256),
                                     ((97, 333), 7), ((500, 64), 32)])
def test_kept_fraction_bounds(shape, P):
    m, n = shape
    W, v = rand_case(m, n, seed=7)
    pr = oracle.probes(W, P)
    N = m * P
    for effort in [0.05, 0.125, 0.25, 0.5, 1.0]:
        r = oracle.run(W, pr, v, effort)
        f = r["total_kept"] / (m * n)
        assert effort <= r["K"] / N + 1e-12
        assert r["K"] / N <= f + 1e-12
        assert f <= r["Kprime"] / N + (-(-n // P) - 1) / n + 1e-12
        # per row: full segments are kept, nothing past the boundary segment is
        for i in range(m):
            mi, ci = int(r["row_chart_kept"][i]), int(r["row_kept"][i])
            assert -(-mi * n // P) <= ci
            if mi < P:
                assert ci <= -(-(mi + 1) * n // P) - 1
            else:
                assert ci == n
        assert r["row_chart_kept"].sum() == r["Kprime"]


# ---------------------------------------------------------------- I4: nesting

def test_nesting_across_efforts():
    W, v = rand_case(256, 256, seed=0, tag="nest")
    pr = oracle.probes(W, 16)
    prev = None
    for effort in [0.01, 0.125, 0.25, 0.5, 0.75, 1.0]:
        r = oracle.run(W, pr, v, effort, mask=True)
        if prev is not None:
            assert r["cutoff"] <= prev["cutoff"]
            assert np.all(r["mask"] >= prev["mask"])
        prev = r


# ---------------------------------------------------------------- I5: layout independence

def test_permutation_invariance():
    W, v = rand_case(64, 96, seed=9)
    rng = np.random.default_rng(9)
    cp = rng.permutation(96)
    rp = rng.permutation(64)
    for effort in [0.25, 0.5]:
        base = oracle.run(W, oracle.probes(W, 8), v, effort, mask=True)
        Wc = np.ascontiguousarray(W[:, cp])
        rc = oracle.run(Wc, oracle.probes(Wc, 8), v, effort, mask=True)
        assert rc["cutoff"] == base["cutoff"]
        assert np.array_equal(rc["mask"], base["mask"][:, cp])
        assert np.array_equal(rc["y"], base["y"][cp])
        Wr = np.ascontiguousarray(W[rp])
        rr = oracle.run(Wr, oracle.probes(Wr, 8), v[rp], effort, mask=True)
        assert rr["cutoff"] == base["cutoff"]
        assert np.array_equal(rr["mask"], base["mask"][rp])
        assert np.allclose(rr["y"], base["y"], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- I6: dropped-mass bound

def test_dropped_mass_bound():
    W, v = rand_case(256, 256, seed=1, tag="drop")
    pr = oracle.probes(W, 16)
    full = oracle.dense(W, v)
    contrib = np.abs(v.astype(np.float64))[:, None] * mags(W)
    for effort in [0.1, 0.25, 0.5]:
        r = oracle.run(W, pr, v, effort, mask=True)
        dropped = r["mask"] == 0
        D = dropped.sum(axis=0)
        mass = np.where(dropped, contrib, 0.0).sum(axis=0)
        err = np.abs(r["y"] - full)
        assert np.all(err <= mass + 1e-12)
        assert np.all(mass[D > 0] < D[D > 0] * float(r["cutoff"]))
        assert np.all(contrib[dropped] < float(r["cutoff"]))


# ---------------------------------------------------------------- I7: scaling and sign

def test_scaling_and_sign():
    W, v = rand_case(128, 200, seed=4, tag="scale")
    pr = oracle.probes(W, 16)
    for effort in [0.25, 0.5]:
        base = oracle.run(W, pr, v, effort, mask=True)
        two = oracle.run(W, pr, (2 * v).astype(np.float32), effort, mask=True)
        assert two["cutoff"] == 2 * base["cutoff"]
        assert np.array_equal(two["mask"], base["mask"])
        assert np.array_equal(two["y"], 2 * base["y"])
        neg = oracle.run(W, pr, -v, effort, mask=True)
        assert neg["cutoff"] == base["cutoff"]
        assert np.array_equal(neg["mask"], base["mask"])
        assert np.array_equal(neg["y"], -base["y"])


# ---------------------------------------------------------------- degenerate inputs

def test_zero_vector_keeps_everything_with_zero_output():
    W, _ = rand_case(16, 24, seed=2)
    pr = oracle.probes(W, 4)
    r = oracle.run(W, pr, np.zeros(16, np.float32), 0.25, mask=True)
    assert r["cutoff"] == 0.0 and r["mask"].all()
    assert np.all(r["y"] == 0.0)


def test_equal_magnitudes_tie_whole_rows():
    W = np.full((8, 12), np.float16(0.5).view(np.uint16), np.uint16)
    W[::2] |= 0x8000  # negative rows
    v = np.linspace(1, 2, 8).astype(np.float32)
    pr = oracle.probes(W, 4)
    r = oracle.run(W, pr, v, 0.3, mask=True)
    # rows are all-or-nothing; the cutoff row and every larger |v_i| row is kept
    kept_rows = r["mask"].all(axis=1)
    assert np.array_equal(kept_rows, r["mask"].any(axis=1))
    assert np.all(np.diff(kept_rows.astype(int)) >= 0)


def test_subnormal_weights_are_exact():
    W = np.array([[0x0001, 0x03FF, 0x8002, 0x0400]], np.uint16)  # subnormals and min normal
    v = np.array([3.0], np.float32)
    pr = oracle.probes(W, 4)
    r = oracle.run(W, pr, v, 1.0, mask=True)
    expect = 3.0 * np.array([2**-24, 1023 * 2**-24, -2 * 2**-24, 2**-14])
    assert np.array_equal(r["y"], expect)
    assert pr[0].tolist() == [2**-14, 1023 * 2**-24, 2 * 2**-24, 2**-24]


# ---------------------------------------------------------------- MON: error vs effort

def test_error_monotone_in_effort_config0():
    """Not a theorem; checked per vector over 20 seeds of the 256 x 256 case."""
    W = synth.matrix("config0", 256, 256, seed=0)
    pr = oracle.probes(W, 16)
    full = oracle.dense(W, synth.vector("config0", 256, seed=0))
    for seed in range(20):
        v = synth.vector("config0", 256, seed=seed)
        full = oracle.dense(W, v)
        errs = [np.linalg.norm(oracle.run(W, pr, v, e)["y"] - full)
                for e in [0.125, 0.25, 0.5, 1.0]]
        assert all(a >= b for a, b in zip(errs, errs[1:])), (seed, errs)
        assert errs[-1] == 0.0


def test_fingerprint_and_counts_follow_the_mask():
    W, v = rand_case(24, 40, seed=8, tag="fp")
    pr = oracle.probes(W, 8)
    r = oracle.run(W, pr, v, 0.3, mask=True)
    ii, jj = np.nonzero(r["mask"])
    fp = 0
    for i, j in zip(ii, jj):
        fp = (fp + synth.splitmix64(int(i) * 40 + int(j))) % 2**64
    assert r["fingerprint"] == fp
    assert np.array_equal(r["row_kept"], r["mask"].sum(axis=1))
    assert r["total_kept"] == len(ii)


# ---------------------------------------------------------------- glue and input generator

def test_silu_mul_identities():
    """silu(x) = x / (1 + e^-x): its odd part is x/2 (so silu(x) - silu(-x) =
    x), silu(0) = 0, silu(ln 3) = ln 3 / (1 + 1/3) = (3/4) ln 3 (a sign error in
    the exponent gives ln 3 / 4), silu(x) -> x for large x, and the gate is
    linear in its second operand."""
    x = np.linspace(-30.0, 30.0, 1201)
    one = np.ones_like(x)
    d = oracle.silu_mul(x, one) - oracle.silu_mul(-x, one)
    assert np.allclose(d, x, rtol=1e-14, atol=1e-14)
    assert oracle.silu_mul(np.array([0.0]), np.array([1.0]))[0] == 0.0
    l3 = math.log(3.0)
    assert abs(oracle.silu_mul(np.array([l3]), np.array([1.0]))[0] - 0.75 * l3) <= 1e-15
    assert abs(oracle.silu_mul(np.array([40.0]), np.array([1.0]))[0] - 40.0) <= 1e-12
    h1 = synth.activations(257, seed=2, stream=3).astype(np.float64)
    h3 = synth.activations(257, seed=4, stream=5).astype(np.float64)
    assert np.array_equal(oracle.silu_mul(h1, 2.0 * h3), 2.0 * oracle.silu_mul(h1, h3))


def test_philox4x32_10_known_answers():
    """Philox4x32-10 against the known-answer vectors published with the
    Random123 library of Salmon, Moraes, Dror and Shaw (SC'11): counter, key,
    expected output."""
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        assert synth.philox4x32_10(ctr, key) == want, (ctr, key)


# ---------------------------------------------------------------- cropped layouts

def _stored_numpy(W, P, crop):
    m, n = W.shape
    keep = -(-crop * n // P)
    st = np.zeros((m, n), np.uint8)
    keys = (W & 0x7FFF).astype(np.int64)
    for i in range(m):
        order = np.lexsort((np.arange(n), -keys[i]))  # key descending, then column ascending
        st[i, order[:keep]] = 1
    return st


@pytest.mark.parametrize("m,n,P,crop", [(40, 300, 16, 12), (9, 37, 5, 2), (5, 64, 64, 63), (3, 20, 4, 4)])
def test_stored_mask_is_top_ranks(m, n, P, crop):
    W, _ = rand_case(m, n, seed=m + crop, tag="crop")
    W[:, ::5] = W[:, 1::5][:, : W[:, ::5].shape[1]] if n > 5 else W[:, ::5]  # ties across columns
    got = oracle.stored_mask(W, P, crop)
    assert np.array_equal(got, _stored_numpy(W, P, crop))
    assert np.all(got.sum(axis=1) == -(-crop * n // P))


def test_run_cropped_reduces_to_run():
    W, v = rand_case(64, 512, seed=1, tag="crop2")
    P = 16
    pr = oracle.probes(W, P)
    for effort in (1.0, 0.3, 0.05):
        full = oracle.run(W, pr, v, effort, mask=True)
        c = oracle.run_cropped(W, pr, v, effort, P, mask=True)  # crop = P stores everything
        for k in ("cutoff", "K", "Kprime", "fingerprint", "total_kept"):
            assert c[k] == full[k], k
        assert np.array_equal(c["mask"], full["mask"]) and np.array_equal(c["y"], full["y"])
        assert not c["crop_reached"]


def test_run_cropped_keeps_stored_part():
    W, v = rand_case(48, 400, seed=2, tag="crop3")
    P, crop = 16, 10
    pr = oracle.probes(W, P)
    st = _stored_numpy(W, P, crop)
    vals = W.view(np.float16).astype(np.float64)
    for effort in (1.0, 0.6, 0.25, 0.02):
        full = oracle.run(W, pr, v, effort, mask=True)
        c = oracle.run_cropped(W, pr, v, effort, crop, mask=True)
        assert c["cutoff"] == full["cutoff"] and c["K"] == full["K"] and c["Kprime"] == full["Kprime"]
        want = full["mask"] & st
        assert np.array_equal(c["mask"], want)
        assert c["crop_reached"] == bool(np.any(full["mask"] & (1 - st)))
        assert np.allclose(c["y"], (v.astype(np.float64)[:, None] * vals * want).sum(axis=0),
                           rtol=1e-12, atol=1e-12)
        if not c["crop_reached"]:  # the kept set lies in the stored part: the uncropped result
            assert c["fingerprint"] == full["fingerprint"] and np.array_equal(c["y"], full["y"])
    # effort 1 keeps every stored pair (no zero activations here) and reaches the crop
    c1 = oracle.run_cropped(W, pr, v, 1.0, crop)
    assert np.all(c1["row_kept"] == -(-crop * 400 // P)) and c1["crop_reached"]
    # a small effort keeps only the largest products, inside the stored part
    assert not oracle.run_cropped(W, pr, v, 0.02, crop)["crop_reached"]


# ---------------------------------------------------------------- Q8 bucketed form

def _q8_brute(W, P):
    """Per row and rank bucket: the 16 levels enumerated from the definition,
    each magnitude key moved to the nearest level by search (ties to the
    upper one)."""
    m, n = W.shape
    out = np.empty_like(W)
    for i in range(m):
        keys = (W[i] & 0x7FFF).astype(np.int64)
        order = np.lexsort((np.arange(n), -keys))
        ends = [-(-(k + 1) * n // P) for k in range(P)]
        start = 0
        for k, end in enumerate(ends):
            lo = keys[order[end - 1]]
            hi = keys[order[0]] if k == 0 else keys[order[start - 1]]
            sh = 0
            while 15 * 2 ** sh < hi - lo:
                sh += 1
            levels = np.minimum(lo + np.arange(16) * 2 ** sh, hi)
            for r in range(start, end):
                j = order[r]
                dist = np.abs(levels - keys[j])
                best = np.flatnonzero(dist == dist.min())[-1]  # ties: the upper level
                out[i, j] = (int(W[i, j]) & 0x8000) | int(levels[best])
            start = end
    return out


@pytest.mark.parametrize("m,n,P", [(6, 200, 16), (4, 37, 5), (3, 64, 64), (5, 33, 1), (2, 1000, 8)])
def test_quantize_q8_against_search(m, n, P):
    W, _ = rand_case(m, n, seed=n + P, tag="q8")
    W[0, ::7] = W[0, 1]        # ties
    W[1 % m, : n // 3] &= 0x83FF  # subnormals
    q = oracle.quantize_q8(W, P)
    assert np.array_equal(q, _q8_brute(W, P))
    assert np.array_equal(q & 0x8000, W & 0x8000)          # signs kept
    assert np.array_equal(oracle.probes(q, P), oracle.probes(W, P))  # buckets' lower ends kept


def test_quantize_q8_properties():
    W, v = rand_case(32, 4096, seed=3, tag="q8p")
    P = 16
    q = oracle.quantize_q8(W, P)
    keys, qk = (W & 0x7FFF).astype(np.int64), (q & 0x7FFF).astype(np.int64)
    # every weight stays inside its bucket: between that bucket's probe and the next larger one
    pr = oracle.probes(W, P).view(np.uint32)  # fp32 bits are monotone in magnitude, like the keys
    assert np.all(qk <= keys.max(axis=1, keepdims=True))
    # at most 16 distinct magnitudes per bucket, so each row uses at most 16 P levels
    for i in range(32):
        assert len(np.unique(qk[i])) <= 16 * P
    # error in key units below half the largest level step of the row
    assert np.all(np.abs(qk - keys) <= keys.max(axis=1, keepdims=True) // 15)
    # the rule on the quantized matrix is a rule like any other: effort 1 is its dense product
    full = oracle.run(q, oracle.probes(q, P), v, 1.0)
    assert np.allclose(full["y"], oracle.dense(q, v), rtol=1e-12, atol=1e-12)
    # quantizing again keeps the grid: levels are fixed points of their own buckets
    assert np.array_equal(oracle.probes(oracle.quantize_q8(q, P), P), oracle.probes(q, P))
    del pr
