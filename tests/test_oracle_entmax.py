"""Pins of the oracle's entmax threshold, probabilities and softmax.

Each check compares the oracle with something other than itself: brute-force
support enumeration, a different algorithm (bisection vs the sort-based closed
forms), hand-derived closed-form values, or textbook limits.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "entmax_closed_forms.json")


def _val(x):
    return float(eval(x, {"sqrt": math.sqrt})) if isinstance(x, str) else float(x)


def _brute_force_tau(z, r):
    """Enumerate every candidate support S; return the tau of the one that is
    self-consistent (all of S above tau, everything else at or below)."""
    n = len(z)
    found = []
    for size in range(1, n + 1):
        for S in itertools.combinations(range(n), size):
            zs = np.array([z[i] for i in S])
            k = len(zs)
            if r == 1:
                t = (zs.sum() - 1.0) / k
            else:
                disc = zs.sum() ** 2 - k * ((zs ** 2).sum() - 1.0)
                if disc < 0:
                    continue
                t = (zs.sum() - math.sqrt(disc)) / k
            rest = [z[i] for i in range(n) if i not in S]
            if zs.min() > t and all(x <= t for x in rest):
                found.append((t, S))
    return found


@pytest.mark.parametrize("alpha,r", [(2.0, 1), (1.5, 2)])
def test_threshold_matches_brute_force_support(alpha, r):
    rng = np.random.default_rng(7)
    for trial in range(150):
        n = int(rng.integers(1, 10))
        z = rng.normal(0, rng.choice([0.3, 1.0, 3.0]), n)
        found = _brute_force_tau(z, r)
        assert len(found) == 1, (z, found)
        t_bf, S = found[0]
        t = O.entmax_threshold(z, alpha)
        assert abs(t - t_bf) < 1e-12
        p = O.entmax_probs(z, t, alpha)
        assert set(np.nonzero(p > 0)[0]) == set(S)


@pytest.mark.parametrize("alpha", [2.0, 1.5])
def test_sort_closed_form_equals_bisection(alpha):
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(1, 400))
        z = rng.normal(0, rng.choice([0.1, 1.0, 5.0]), n)
        t1 = O.entmax_threshold(z, alpha)
        t2 = O.entmax_threshold_bisect(z, alpha)
        assert abs(t1 - t2) < 1e-11


@pytest.mark.parametrize("alpha", [2.0, 1.5, 1.25, 1.75, 3.0])
def test_invariants(alpha):
    rng = np.random.default_rng(3)
    for trial in range(100):
        n = int(rng.integers(1, 300))
        z = rng.normal(0, 2.0, n)
        t = O.entmax_threshold(z, alpha)
        p = O.entmax_probs(z, t, alpha)
        assert abs(p.sum() - 1.0) < 1e-10
        assert (p >= 0).all()
        assert ((p > 0) == (z > t)).all()
        zmax = z.max()
        assert zmax - 1.0 - 1e-12 <= t <= zmax - n ** (-(alpha - 1)) + 1e-12


def test_golden_closed_forms():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        z = np.array(c["z"], dtype=np.float64)
        t = O.entmax_threshold(z, c["alpha"])
        p = O.entmax_probs(z, t, c["alpha"])
        assert abs(t - _val(c["tau"])) < 1e-12, c
        np.testing.assert_allclose(p, [_val(x) for x in c["p"]], atol=1e-12)


def test_two_point_closed_forms():
    # sparsemax([a, b]) puts clip((a - b + 1)/2, 0, 1) on a; 1.5-entmax puts
    # ((1 + d)/2 + ... ) -- derived: both in support iff |d| < 1, then
    # (a-t)^2 + (b-t)^2 = 1 with d = a - b gives p_a = ((d + sqrt(2 - d^2))/2)^2.
    for d in np.linspace(-1.5, 1.5, 61):
        z = np.array([d, 0.0])
        t = O.entmax_threshold(z, 2.0)
        p = O.entmax_probs(z, t, 2.0)
        assert abs(p[0] - min(max((d + 1) / 2, 0), 1)) < 1e-12
        t = O.entmax_threshold(z, 1.5)
        p = O.entmax_probs(z, t, 1.5)
        if abs(d) < 1:
            expect = ((d + math.sqrt(2 - d * d)) / 2) ** 2
        else:
            expect = 1.0 if d > 0 else 0.0
        assert abs(p[0] - expect) < 1e-12


def test_attend_is_weighted_value_sum():
    rng = np.random.default_rng(5)
    K = rng.normal(size=(50, 8))
    V = rng.normal(size=(50, 8))
    q = rng.normal(size=8) * 2
    o, t, p = O.entmax_attend(q, K, V, 0.5, 1.5)
    z = 0.5 * 0.5 * (K @ q)
    assert abs(O.entmax_threshold(z, 1.5) - t) < 1e-14
    np.testing.assert_allclose(o, (p[:, None] * V).sum(0), atol=1e-12)


def test_softmax_two_token_and_shift():
    rng = np.random.default_rng(9)
    for _ in range(20):
        K = rng.normal(size=(2, 4))
        V = rng.normal(size=(2, 4))
        q = rng.normal(size=4)
        o, lse = O.softmax_attend(q, K, V, 1.0)
        s = K @ q
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))  # logistic form
        np.testing.assert_allclose(o, w0 * V[0] + (1 - w0) * V[1], atol=1e-12)
        assert abs(lse - (max(s) + math.log1p(math.exp(-abs(s[0] - s[1]))))) < 1e-12
    K = rng.normal(size=(30, 4))
    V = rng.normal(size=(30, 4))
    q = rng.normal(size=4)
    o1, l1 = O.softmax_attend(q, K, V, 1.0)
    # adding a constant key component along q shifts every score equally
    shift = np.outer(np.ones(30), q / (q @ q)) * 3.0
    o2, l2 = O.softmax_attend(q, K + shift, V, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    assert abs((l2 - l1) - 3.0) < 1e-12


def test_entmax_tends_to_softmax_as_alpha_to_one():
    rng = np.random.default_rng(13)
    K = rng.normal(size=(40, 6))
    V = rng.normal(size=(40, 6))
    q = rng.normal(size=6)
    o_sm, _ = O.softmax_attend(q, K, V, 1.0)
    alpha = 1.0005
    z = (alpha - 1) * (K @ q)
    t = O.entmax_threshold_bisect(z, alpha, tol=1e-18)
    p = O.entmax_probs(z, t, alpha)
    o_em = (p[:, None] * V).sum(0) / p.sum()
    np.testing.assert_allclose(o_em, o_sm, atol=5e-3)


def test_support_recovery_is_exact_and_error_bound_holds():
    # Technical Summary, §3: a kept set containing the support loses nothing;
    # any kept set errs by at most 2 B delta.
    rng = np.random.default_rng(17)
    for alpha in (1.5, 2.0):
        K = rng.normal(size=(300, 16))
        V = rng.normal(size=(300, 16))
        q = rng.normal(size=16) * 1.5
        o_full, t_full, p_full = O.entmax_attend(q, K, V, 0.25, alpha)
        supp = np.nonzero(p_full > 0)[0]
        extra = rng.choice(300, 40, replace=False)
        kept = np.union1d(supp, extra)
        o_k, t_k, _ = O.entmax_attend(q, K[kept], V[kept], 0.25, alpha)
        assert t_k == t_full
        assert np.array_equal(o_k, o_full)
        Bv = np.linalg.norm(V, axis=1).max()
        worst = 0.0
        for _ in range(100):
            kept = np.sort(rng.choice(300, int(rng.integers(1, 300)), replace=False))
            delta, _, _ = O.dropped_mass(q, K, kept, 0.25, alpha)
            o_k, _, _ = O.entmax_attend(q, K[kept], V[kept], 0.25, alpha)
            err = np.linalg.norm(o_k - o_full)
            assert err <= 2 * Bv * delta + 1e-12
            if delta > 0:
                worst = max(worst, err / (2 * Bv * delta))
        assert worst > 0.0


def test_softmax_dropped_mass_two_tokens():
    # scores 0 and ln 3 (scale 1, unit vectors): weights 1/4 and 3/4
    K = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    q = np.array([1.0, 0.0])
    assert abs(O.softmax_dropped_mass(q, K, [0], 1.0) - 0.75) < 1e-15
    assert abs(O.softmax_dropped_mass(q, K, [1], 1.0) - 0.25) < 1e-15
    assert O.softmax_dropped_mass(q, K, [0, 1], 1.0) == 0.0


def test_softmax_dropped_mass_equals_lse_gap():
    # mass outside = 1 - exp(lse(kept) - lse(all)), two independent routes
    rng = np.random.default_rng(41)
    K = rng.normal(size=(500, 32))
    V = rng.normal(size=(500, 32))
    for _ in range(20):
        q = rng.normal(size=32) * 2.0
        kept = np.sort(rng.choice(500, int(rng.integers(1, 500)), replace=False))
        _, l_all = O.softmax_attend(q, K, V, 0.3)
        _, l_kept = O.softmax_attend(q, K[kept], V[kept], 0.3)
        d = O.softmax_dropped_mass(q, K, kept, 0.3)
        assert abs(d - (1.0 - math.exp(l_kept - l_all))) < 1e-12


def test_support_recall_cases():
    p = np.array([0.0, 0.5, 0.0, 0.3, 0.2, 0.0])
    assert O.support_recall(p, [1, 3, 4]) == 1.0
    assert O.support_recall(p, [0, 2, 5]) == 0.0
    assert abs(O.support_recall(p, [1, 2]) - 1.0 / 3.0) < 1e-15


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_matched_budget_quality(alpha):
    rng = np.random.default_rng(43)
    P, N, D = 16, 16 * 40 - 5, 16
    K = rng.normal(size=(N, D))
    K[100:140] += 2.0 * rng.normal(size=D)  # one page run the queries align with
    V = rng.normal(size=(N, D))
    qs = np.stack([K[120] * 0.05, K[130] * 0.05])  # supports over pages 6-8
    sc = 0.5
    # every page: nothing dropped, the full-cache outputs
    allp = np.arange((N + P - 1) // P)
    m = O.matched_budget_quality(qs, K, V, P, sc, alpha, allp)
    assert (m["delta_entmax"] == 0).all() and (m["delta_softmax"] == 0).all()
    assert (m["recall"] == 1).all()
    assert (m["err_entmax"] < 1e-12).all() and (m["err_softmax"] < 1e-12).all()
    # the pages holding each head's support: entmax exact, softmax not
    supp_pages = set()
    for q in qs:
        _, p, _ = O.dropped_mass(q, K, [], sc, alpha)
        supp_pages |= set((np.flatnonzero(p > 0) // P).tolist())
    pages = np.array(sorted(supp_pages))
    assert len(pages) < len(allp)
    m = O.matched_budget_quality(qs, K, V, P, sc, alpha, pages)
    assert (m["delta_entmax"] == 0).all() and (m["recall"] == 1).all()
    assert (m["err_entmax"] < 1e-12).all()
    assert (m["delta_softmax"] > 0).all() and (m["err_softmax"] > 0).all()
    # a set missing part of the support: error within 2 B delta
    Bv = np.linalg.norm(V, axis=1).max()
    m = O.matched_budget_quality(qs, K, V, P, sc, alpha, pages[: len(pages) // 2])
    for h, q in enumerate(qs):
        _, p, _ = O.dropped_mass(q, K, [], sc, alpha)
        o_full = p @ V
        assert m["delta_entmax"][h] > 0 and m["recall"][h] < 1
        assert m["err_entmax"][h] * np.linalg.norm(o_full) <= 2 * Bv * m["delta_entmax"][h] + 1e-12
