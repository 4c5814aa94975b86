"""Host-side glue of chained matvecs: expert routing."""
import itertools
import math

import numpy as np
import pytest

import dynamic_sparsity_approximate_amd as E


def brute_top2(logits):
    # every ordered pair, best by (larger first logit, then larger second, then lower indices)
    best = None
    for e0, e1 in itertools.permutations(range(len(logits)), 2):
        ok = all(logits[e0] > logits[k] or (logits[e0] == logits[k] and e0 <= k)
                 for k in range(len(logits)))
        rest = [k for k in range(len(logits)) if k != e0]
        ok2 = all(logits[e1] > logits[k] or (logits[e1] == logits[k] and e1 <= k) for k in rest)
        if ok and ok2:
            best = (e0, e1)
    return best


@pytest.mark.parametrize("seed", range(20))
def test_route_top2_random(seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(8).astype(np.float32)
    e0, e1, g0, g1 = E.route_top2(logits)
    assert (e0, e1) == brute_top2(list(logits))
    a, b = float(logits[e0]), float(logits[e1])
    assert math.isclose(g0, math.exp(a) / (math.exp(a) + math.exp(b)), rel_tol=1e-12)
    assert math.isclose(g0 + g1, 1.0, rel_tol=1e-12) and g0 >= g1


def test_route_top2_ties_and_shift():
    e0, e1, g0, g1 = E.route_top2([1.0, 3.0, 3.0, 0.0])
    assert (e0, e1) == (1, 2) and g0 == g1 == 0.5
    # softmax over the pair is invariant to a common shift
    r1 = E.route_top2([0.1, 2.0, -1.0, 1.5])
    r2 = E.route_top2([100.1, 102.0, 99.0, 101.5])
    assert r1[:2] == r2[:2] and math.isclose(r1[2], r2[2], rel_tol=1e-9)


def test_effort_schedule_lookup_order():
    from dynamic_sparsity_approximate_amd import EffortSchedule
    s = EffortSchedule(0.25, {(3, "wq"): 0.5, (None, "w2"): 0.125, (7, None): 0.75})
    assert s(3, "wq") == 0.5          # (unit, role)
    assert s(3, "w2") == 0.125        # (None, role) before (unit, None)
    assert s(7, "w2") == 0.125
    assert s(7, "wk") == 0.75         # (unit, None)
    assert s(0, "wk") == 0.25         # default
    a = EffortSchedule.from_array([[0.1] * 7, [0.3] * 7], head=0.9)
    assert a(1, "w1") == 0.3 and a(None, "head") == 0.9 and abs(a.default - 0.2) < 1e-12


def test_effort_schedule_rejects_bad_efforts():
    from dynamic_sparsity_approximate_amd import EffortSchedule
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            EffortSchedule(bad)
        with pytest.raises(ValueError):
            EffortSchedule(0.5, {(0, "wq"): bad})
    with pytest.raises(ValueError):
        EffortSchedule.from_array([[0.5, 0.5]])
