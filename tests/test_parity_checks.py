"""The selection checks of the GPU parity tests accept exactly the allowed
differences: pages within the cutoff tolerance, and the Gaussian selector's
single-page fallback when it picks the page with the largest margin.  Each
case plants a GPU result on the CPU; no GPU is used."""
import math

import numpy as np
import pytest

import oracle as O
from parity_utils import CUT_REL, check_gauss_selection, check_topk_selection


def _gauss_case(seed=5, G=3, n=40, P=16):
    rng = np.random.default_rng(seed)
    mu = rng.normal(size=(G, n)) * 2.0
    s2 = rng.uniform(0.05, 0.4, size=(G, n))
    n_tok = np.full(n, P)
    n_tok[-1] = 5
    alpha, delta = 1.5, 0.5
    th = np.array([O.solve_tau_hat(mu[h], s2[h], n_tok, alpha) for h in range(G)])
    return mu, s2, n_tok, th, alpha, delta


def test_gauss_check_accepts_the_oracle_set_and_rejects_a_planted_single_page():
    mu, s2, n_tok, th, alpha, delta = _gauss_case()
    ref = O.gauss_keep(mu, s2, n_tok, th, alpha, delta)
    assert len(ref) > 3
    assert check_gauss_selection(ref, mu, s2, n_tok, th, alpha, delta) == 0
    # a GPU that fell back to one page while the oracle keeps many
    for p in (int(ref[0]), int(ref[-1])):
        with pytest.raises(AssertionError):
            check_gauss_selection([p], mu, s2, n_tok, th, alpha, delta)
    # a page dropped or added far from every cut
    with pytest.raises(AssertionError):
        check_gauss_selection(ref[1:], mu, s2, n_tok, th, alpha, delta)
    G = mu.shape[0]
    zhat = np.stack([(alpha - 1) * O.page_max_estimate(mu[h], s2[h], n_tok)
                     for h in range(G)])
    far = [p for p in range(mu.shape[1]) if p not in set(ref.tolist())
           and np.all(zhat[:, p] < th - delta - 0.1)]
    assert far
    with pytest.raises(AssertionError):
        check_gauss_selection(sorted(set(ref.tolist()) | {far[0]}), mu, s2,
                              n_tok, th, alpha, delta)


def test_gauss_check_accepts_a_near_cut_swap():
    mu, s2, n_tok, th, alpha, delta = _gauss_case(seed=6)
    ref = set(O.gauss_keep(mu, s2, n_tok, th, alpha, delta).tolist())
    # move page 7's estimate for head 0 onto the cut, just above it
    p, h = 7, 0
    c = math.sqrt(2.0 * math.log(n_tok[p]))
    sd = math.sqrt(s2[h, p])
    mu = mu.copy()
    for hh in range(mu.shape[0]):  # keep the other heads far below their cuts
        if hh != h:
            mu[hh, p] = (th[hh] - delta - 1.0) / (alpha - 1) - c * math.sqrt(s2[hh, p])
    mu[h, p] = (th[h] - delta) / (alpha - 1) - c * sd + 1e-9
    ref = set(O.gauss_keep(mu, s2, n_tok, th, alpha, delta).tolist())
    assert p in ref
    assert check_gauss_selection(sorted(ref - {p}), mu, s2, n_tok, th, alpha,
                                 delta) == 1


def test_gauss_check_fallback_page_must_have_the_largest_margin():
    # many pages of the same wide Gaussian: the normaliser is reached in the
    # tail, past every page's estimated maximum, so no page clears its cut
    G, n, P = 2, 200, 16
    rng = np.random.default_rng(9)
    mu = rng.normal(size=(G, n)) * 0.01
    s2 = np.full((G, n), 1.0)
    n_tok = np.full(n, P)
    alpha, delta = 1.5, 0.0
    th = np.array([O.solve_tau_hat(mu[h], s2[h], n_tok, alpha) for h in range(G)])
    ref = O.gauss_keep(mu, s2, n_tok, th, alpha, delta)
    assert len(ref) == 1  # nothing clears its cut: the fallback page
    assert check_gauss_selection(ref, mu, s2, n_tok, th, alpha, delta) == 0
    other = (int(ref[0]) + 5) % n
    with pytest.raises(AssertionError):
        check_gauss_selection([other], mu, s2, n_tok, th, alpha, delta)
    # a page tied with the best margin is an equally valid fallback
    mu2 = mu.copy()
    mu2[:, other] = mu2[:, int(ref[0])]
    ref2 = O.gauss_keep(mu2, s2, n_tok, th, alpha, delta)
    assert len(ref2) == 1
    assert check_gauss_selection([other], mu2, s2, n_tok, th, alpha, delta) == 2


def test_topk_check_accepts_near_ties_only():
    rng = np.random.default_rng(3)
    G, D, P, N, k = 2, 8, 4, 4 * 30, 5
    qs = rng.normal(size=(G, D))
    keys = rng.normal(size=(N, D))
    ref = O.decode_unit(qs, keys, rng.normal(size=(N, D)), P, 0.5, 1.5,
                        "topk", k=k)
    sel = ref["sel"].tolist()
    assert check_topk_selection(sel, ref, k) == 0
    g = ref["g"]
    order = sorted(range(len(g)), key=lambda p: (-g[p], p))
    # the (k+1)-th page instead of the k-th: allowed only when they nearly tie
    swapped = sorted(set(sel) - {order[k - 1]} | {order[k]})
    if abs(g[order[k]] - g[order[k - 1]]) > CUT_REL * max(abs(g[order[k - 1]]), 1.0):
        with pytest.raises(AssertionError):
            check_topk_selection(swapped, ref, k)
    near = dict(ref)
    near["g"] = g.copy()
    near["g"][order[k]] = g[order[k - 1]] * (1 - 1e-7)
    assert check_topk_selection(swapped, near, k) == 2
    with pytest.raises(AssertionError):
        check_topk_selection(sel[:-1], ref, k)
