"""Pins of the oracle's page metadata, page scores and the two selectors."""
import itertools
import math

import numpy as np
import pytest
from scipy import integrate

import oracle as O


# --- metadata -----------------------------------------------------------------

def test_metadata_identities():
    rng = np.random.default_rng(1)
    for n in (1, 2, 7, 64):
        keys = rng.normal(size=(n, 12)) * 3 + 1
        kmin, kmax, mean, var = O.page_metadata(keys)
        assert (kmin <= mean + 1e-12).all() and (mean <= kmax + 1e-12).all()
        assert (var >= 0).all()
        # one-pass second-moment form
        np.testing.assert_allclose(var, (keys ** 2).mean(0) - mean ** 2,
                                   atol=1e-10)
        # translation moves the box and the mean, not the variance
        c = rng.normal(size=12)
        kmin2, kmax2, mean2, var2 = O.page_metadata(keys + c)
        np.testing.assert_allclose(kmin2, kmin + c, atol=1e-12)
        np.testing.assert_allclose(kmax2, kmax + c, atol=1e-12)
        np.testing.assert_allclose(mean2, mean + c, atol=1e-12)
        np.testing.assert_allclose(var2, var, atol=1e-10)
    k1 = rng.normal(size=(1, 5))
    kmin, kmax, mean, var = O.page_metadata(k1)
    assert (kmin == k1[0]).all() and (kmax == k1[0]).all()
    assert (mean == k1[0]).all() and (var == 0).all()


def test_unit_metadata_partial_last_page():
    rng = np.random.default_rng(2)
    keys = rng.normal(size=(37, 4))
    kmin, kmax, mean, var = O.unit_metadata(keys, 16)
    assert kmin.shape == (3, 4)
    assert np.array_equal(kmin[2], keys[32:].min(0))
    assert np.allclose(mean[2], keys[32:].mean(0))
    assert list(O.page_token_counts(37, 16)) == [16, 16, 5]


# --- page scores ----------------------------------------------------------------

def test_bbox_bound_equals_best_box_corner():
    # The largest score over the box is attained at a corner: enumerate all.
    rng = np.random.default_rng(3)
    for _ in range(30):
        D = 6
        keys = rng.normal(size=(5, D))
        q = rng.normal(size=D)
        kmin, kmax, _, _ = O.page_metadata(keys)
        ub = O.bbox_bound(q, kmin[None], kmax[None], 0.7)[0]
        best = max(0.7 * float(np.dot(q, np.where(c, kmax, kmin)))
                   for c in itertools.product([0, 1], repeat=D))
        assert abs(ub - best) < 1e-12
        assert ub >= 0.7 * (keys @ q).max() - 1e-12


def test_bbox_bound_sign_split_and_single_token():
    rng = np.random.default_rng(4)
    keys = rng.normal(size=(100, 32))
    q = rng.normal(size=32)
    kmin, kmax, _, _ = O.unit_metadata(keys, 10)
    ub = O.bbox_bound(q, kmin, kmax, 0.3)
    split = 0.3 * (kmax @ np.maximum(q, 0) + kmin @ np.minimum(q, 0))
    np.testing.assert_allclose(ub, split, atol=1e-12)
    s = O.token_scores(q, keys, 0.3)
    for p in range(10):
        assert ub[p] >= s[p * 10:(p + 1) * 10].max() - 1e-12
    # pages of one token: the bound is the score itself
    kmin1, kmax1, _, _ = O.unit_metadata(keys, 1)
    np.testing.assert_allclose(O.bbox_bound(q, kmin1, kmax1, 0.3), s, atol=1e-12)


def test_gauss_moments_one_coordinate_is_exact():
    # With one coordinate the page's scores are q*scale*k exactly, so their
    # mean and population variance are the Gaussian moments.
    rng = np.random.default_rng(5)
    keys = rng.normal(size=(64, 1)) * 2 + 1
    q = np.array([1.7])
    _, _, mean, var = O.page_metadata(keys)
    mu, s2 = O.gauss_moments(q, mean[None], var[None], 0.5)
    s = O.token_scores(q, keys, 0.5)
    assert abs(mu[0] - s.mean()) < 1e-12
    assert abs(s2[0] - s.var()) < 1e-12


def test_gauss_moments_monte_carlo():
    rng = np.random.default_rng(6)
    D = 16
    mean = rng.normal(size=D)
    var = rng.uniform(0.1, 2.0, D)
    q = rng.normal(size=D)
    mu, s2 = O.gauss_moments(q, mean[None], var[None], 0.25)
    keys = mean + np.sqrt(var) * rng.normal(size=(400000, D))
    s = O.token_scores(q, keys, 0.25)
    assert abs(s.mean() - mu[0]) < 4 * math.sqrt(s2[0] / 400000)
    assert abs(s.var() / s2[0] - 1) < 0.02


# --- top-k ----------------------------------------------------------------------

def test_topk_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        g = rng.integers(-3, 4, n).astype(float)  # many ties on purpose
        k = int(rng.integers(1, 10))
        sel = O.select_topk(g, k)
        m = min(k, n)
        # best subset: largest sum of g, then the smallest sorted index list
        best = min(itertools.combinations(range(n), m),
                   key=lambda S: (-sum(g[list(S)]), sorted(S)))
        assert list(sel) == sorted(best)


def test_topk_nesting_and_all():
    rng = np.random.default_rng(8)
    g = rng.normal(size=50)
    prev = set()
    for k in range(1, 51):
        cur = set(O.select_topk(g, k))
        assert prev <= cur and len(cur) == k
        prev = cur
    assert list(O.select_topk(g, 80)) == list(range(50))


def test_group_bound_on_one_token_pages_is_the_best_head_score():
    """With one token per page each head's box is a point, so the group's
    ranking value must be the largest exact score over the query heads and
    top-k must keep the pages of the k largest of those."""
    rng = np.random.default_rng(81)
    G, D, N, k = 4, 8, 40, 6
    scale = 1.0 / math.sqrt(D)
    for _ in range(5):
        qs = rng.normal(size=(G, D)) * rng.uniform(0.2, 3.0, size=(G, 1))
        keys = rng.normal(size=(N, D))
        vals = rng.normal(size=(N, D))
        res = O.decode_unit(qs, keys, vals, 1, scale, 1.5, "topk", k=k)
        best = np.array([max(scale * sum(qs[h, d] * keys[i, d] for d in range(D))
                             for h in range(G)) for i in range(N)])
        np.testing.assert_allclose(res["g"], best, rtol=1e-12, atol=1e-12)
        order = sorted(range(N), key=lambda i: (-best[i], i))
        assert list(res["sel"]) == sorted(order[:k])


def test_group_bound_bounds_every_head_and_is_attained():
    """On pages of many tokens the group value bounds the score of every
    token of the page for every query head of the group, and it is one of
    the heads' own box bounds (the tightest value with that property)."""
    rng = np.random.default_rng(82)
    G, D, P, N = 4, 16, 16, 16 * 12 + 5
    scale = 1.0 / math.sqrt(D)
    qs = rng.normal(size=(G, D)) * np.array([[0.3], [1.0], [2.0], [0.7]])
    keys = rng.normal(size=(N, D))
    # needles aligned to the last head only, in pages 3 and 8
    for i in (3 * P + 2, 8 * P + 11):
        keys[i] = 3.0 * qs[G - 1] / np.linalg.norm(qs[G - 1])
    res = O.decode_unit(qs, keys, rng.normal(size=(N, D)), P, scale, 1.5,
                        "topk", k=4)
    g, ub = res["g"], res["ub"]
    for p in range(len(g)):
        toks = range(p * P, min((p + 1) * P, N))
        top = max(scale * float(np.dot(qs[h], keys[i])) for h in range(G) for i in toks)
        assert g[p] >= top - 1e-12
        assert any(g[p] == ub[h, p] for h in range(G))
        assert all(g[p] >= ub[h, p] for h in range(G))
    assert {3, 8} <= set(res["sel"].tolist())


# --- Gaussian expectation and threshold estimate ---------------------------------

@pytest.mark.parametrize("r", [1, 2])
def test_gauss_excess_moment_quadrature(r):
    for m, s, tau in [(0.0, 1.0, 0.0), (2.0, 0.3, 1.5), (-1.0, 0.5, 0.7),
                      (5.0, 2.0, -1.0), (0.1, 0.05, 0.3)]:
        f = lambda x: max(x - tau, 0.0) ** r * math.exp(
            -0.5 * ((x - m) / s) ** 2) / (s * math.sqrt(2 * math.pi))
        val, _ = integrate.quad(f, tau, m + 40 * s + abs(tau) + 10, limit=400,
                                epsabs=1e-14, epsrel=1e-12)
        got = float(O.gauss_excess_moment(m, s, tau, r))
        assert abs(got - val) < 1e-10 * max(1.0, val)


def test_gauss_excess_moment_monte_carlo_and_zero_variance():
    rng = np.random.default_rng(9)
    x = rng.normal(1.2, 0.7, 2_000_000)
    for r in (1, 2):
        mc = np.mean(np.maximum(x - 1.0, 0) ** r)
        assert abs(float(O.gauss_excess_moment(1.2, 0.7, 1.0, r)) - mc) < 1e-2 * mc + 1e-3
        assert float(O.gauss_excess_moment(1.2, 0.0, 1.0, r)) == pytest.approx(0.2 ** r)
        assert float(O.gauss_excess_moment(1.2, 0.0, 1.5, r)) == 0.0


def _phi(c):
    return math.exp(-0.5 * c * c) / math.sqrt(2 * math.pi)


def _Q(c):
    return 0.5 * math.erfc(c / math.sqrt(2))


@pytest.mark.parametrize("c", [-45.0, -31.0, -29.0, -12.0, -3.0, -0.5, 0.0, 1.7, 6.0, 10.0])
def test_excess_standard_matches_closed_forms(c):
    # parabolic-cylinder form (and the series far below) against the
    # elementary closed forms at r = 1, 2
    j1 = _phi(c) - c * _Q(c)
    j2 = (1 + c * c) * _Q(c) - c * _phi(c)
    assert abs(float(O.excess_standard(c, 1.0)) - j1) <= 1e-11 * max(abs(j1), 1e-300)
    assert abs(float(O.excess_standard(c, 2.0)) - j2) <= 1e-10 * max(abs(j2), 1e-300)


@pytest.mark.parametrize("r", [4.0 / 3.0, 3.0, 4.0, 7.5])
def test_excess_standard_quadrature(r):
    # the defining integral J_r(c) = int_c^inf (x - c)^r phi(x) dx
    for c in (-40.0, -31.0, -29.0, -10.0, -3.0, 0.0, 2.0, 6.0, 10.0):
        f = lambda x: (x - c) ** r * _phi(x)
        lo = max(c, -40.0)
        val = sum(integrate.quad(f, a, b, limit=400, epsabs=0, epsrel=1e-13)[0]
                  for a, b in ((lo, lo + 5), (lo + 5, max(lo + 5, 12.0) + 30)))
        got = float(O.excess_standard(c, r))
        assert abs(got - val) <= 1e-8 * val, (r, c, got, val)


@pytest.mark.parametrize("r", [3.25, 4.5])
def test_excess_standard_recurrence(r):
    # integration by parts: J_r = (r - 1) J_(r-2) - c J_(r-1)
    for c in (-20.0, -2.0, 0.0, 1.0, 4.0):
        jr, j1, j2 = (float(O.excess_standard(c, x)) for x in (r, r - 1, r - 2))
        assert abs(jr - ((r - 1) * j2 - c * j1)) <= 1e-9 * abs(jr)


def test_gauss_excess_moment_general_r_monte_carlo():
    rng = np.random.default_rng(19)
    x = rng.normal(0.4, 0.9, 4_000_000)
    for r in (4.0 / 3.0, 4.0):
        mc = np.mean(np.maximum(x - 0.1, 0) ** r)
        got = float(O.gauss_excess_moment(0.4, 0.9, 0.1, r))
        assert abs(got - mc) < 5e-3 * mc
        assert float(O.gauss_excess_moment(0.4, 0.0, 0.1, r)) == pytest.approx(0.3 ** r)


@pytest.mark.parametrize("alpha", [1.25, 1.75])
def test_tau_hat_zero_variance_general_alpha(alpha):
    # zero variance: the normalisation is the exact entmax one over the
    # repeated page means (bisection threshold for these alpha)
    rng = np.random.default_rng(11)
    for _ in range(10):
        n_pages = int(rng.integers(1, 30))
        mu = rng.normal(0, 2, n_pages)
        n_tok = rng.integers(1, 17, n_pages)
        th = O.solve_tau_hat(mu, np.zeros(n_pages), n_tok, alpha)
        z = np.repeat((alpha - 1) * mu, n_tok)
        assert abs(th - O.entmax_threshold_bisect(z, alpha)) < 1e-9


@pytest.mark.parametrize("alpha", [1.25, 1.75])
def test_tau_hat_general_alpha_is_the_unique_root(alpha):
    rng = np.random.default_rng(14)
    r = 1 / (alpha - 1)
    for _ in range(10):
        n_pages = int(rng.integers(1, 150))
        mu = rng.normal(0, 3, n_pages)
        s2 = rng.uniform(0, 1.5, n_pages)
        n_tok = np.full(n_pages, 32)
        th = O.solve_tau_hat(mu, s2, n_tok, alpha)
        m, s = (alpha - 1) * mu, (alpha - 1) * np.sqrt(s2)
        assert abs(O.gauss_normaliser(th, m, s, n_tok, r) - 1.0) < 1e-9
        assert O.gauss_normaliser(th - 1e-6, m, s, n_tok, r) > 1.0
        assert O.gauss_normaliser(th + 1e-6, m, s, n_tok, r) < 1.0


def test_solve_tau_hat_rejects_alpha_above_two():
    with pytest.raises(ValueError):
        O.solve_tau_hat(np.zeros(3), np.ones(3), np.full(3, 8), 2.5)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_tau_hat_zero_variance_is_exact_threshold(alpha):
    # With zero page variance every token of page p scores mu_p, so the
    # normalisation is the exact entmax one over mu_p repeated n_p times.
    rng = np.random.default_rng(10)
    for _ in range(20):
        n_pages = int(rng.integers(1, 40))
        mu = rng.normal(0, 2, n_pages)
        n_tok = rng.integers(1, 17, n_pages)
        th = O.solve_tau_hat(mu, np.zeros(n_pages), n_tok, alpha)
        z = np.repeat((alpha - 1) * mu, n_tok)
        assert abs(th - O.entmax_threshold(z, alpha)) < 1e-10


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_tau_hat_is_the_unique_root(alpha):
    rng = np.random.default_rng(12)
    r = 1 if alpha == 2.0 else 2
    for _ in range(20):
        n_pages = int(rng.integers(1, 200))
        mu = rng.normal(0, 3, n_pages)
        s2 = rng.uniform(0, 1.5, n_pages)
        n_tok = np.full(n_pages, 32)
        th = O.solve_tau_hat(mu, s2, n_tok, alpha)
        m, s = (alpha - 1) * mu, (alpha - 1) * np.sqrt(s2)
        assert abs(O.gauss_normaliser(th, m, s, n_tok, r) - 1.0) < 1e-9
        assert O.gauss_normaliser(th - 1e-6, m, s, n_tok, r) > 1.0
        assert O.gauss_normaliser(th + 1e-6, m, s, n_tok, r) < 1.0
        assert th >= m.max() - 1.0


def test_page_max_estimate_bounds_the_expected_maximum():
    # mu + sigma sqrt(2 ln n) is the classical upper bound on the expected
    # largest of n draws of N(mu, sigma^2); it is exact at n = 1 and, measured
    # above mu, within 35 % of the expected maximum at n = 16 and 64 (the
    # bound tightens as n grows).  Checked against Monte Carlo maxima.
    rng = np.random.default_rng(17)
    mu, s2 = np.array([0.3]), np.array([2.25])
    assert O.page_max_estimate(mu, s2, np.array([1]))[0] == pytest.approx(0.3)
    for n in (2, 16, 64):
        est = O.page_max_estimate(mu, s2, np.array([n]))[0]
        mc = (0.3 + 1.5 * rng.standard_normal((200000, n))).max(axis=1).mean()
        assert est >= mc
        if n >= 16:
            assert (est - 0.3) <= 1.35 * (mc - 0.3)


def test_gauss_keep_limits():
    rng = np.random.default_rng(13)
    G, n = 4, 60
    mu = rng.normal(size=(G, n))
    s2 = rng.uniform(0, 0.5, (G, n))
    n_tok = np.full(n, 16)
    th = np.array([O.solve_tau_hat(mu[h], s2[h], n_tok, 1.5) for h in range(G)])
    assert list(O.gauss_keep(mu, s2, n_tok, th, 1.5, math.inf)) == list(range(n))
    # a threshold above every estimate keeps exactly the best-margin page
    big = th + 100.0
    kept = O.gauss_keep(mu, s2, n_tok, big, 1.5, 0.0)
    zhat = np.stack([0.5 * O.page_max_estimate(mu[h], s2[h], n_tok) for h in range(G)])
    assert list(kept) == [int(np.argmax((zhat - big[:, None]).max(0)))]


def test_gauss_selector_recovers_support_on_single_token_pages():
    # One-token pages have zero variance and mhat = mu = the token's score:
    # with delta -> 0+ the kept pages are exactly the entmax support.
    rng = np.random.default_rng(14)
    keys = rng.normal(size=(200, 8))
    vals = rng.normal(size=(200, 8))
    qs = rng.normal(size=(1, 8)) * 2
    res = O.decode_unit(qs, keys, vals, 1, 0.5, 1.5, "gauss", delta=1e-12)
    full = O.decode_unit(qs, keys, vals, 1, 0.5, 1.5, "full")
    z = 0.5 * O.token_scores(qs[0], keys, 0.5)
    supp = np.nonzero(z > full["tau"][0])[0]
    assert abs(res["tau_hat"][0] - full["tau"][0]) < 1e-10
    assert list(res["sel"]) == list(supp)
    assert np.array_equal(res["out"], full["out"])


def test_unit_tokens_round_trip():
    # Logical token i of a sequence lives at offset i % P of the physical
    # slot the page table names for page i // P.  Scattering numbered tokens
    # into a pool by that rule, with a random page table, two KV heads and a
    # short last page, the gather must give them back in order.
    rng = np.random.default_rng(23)
    P, D, H, n = 4, 3, 2, 13
    n_pages = (n + P - 1) // P
    table = rng.permutation(7)[:n_pages]
    pool = rng.standard_normal((7, H, P, D))
    seq = np.arange(n * D, dtype=np.float64).reshape(n, D)
    for i in range(n):
        pool[table[i // P], 1, i % P] = seq[i]
    np.testing.assert_array_equal(O.unit_tokens(pool, table, 1, n), seq)
    assert not np.array_equal(O.unit_tokens(pool, table, 0, n), seq)


def test_bf16_decoding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625
    assert math.copysign(1.0, vals[4]) == -1.0
    assert vals[5] == (2 - 2 ** -7) * 2.0 ** 127
