"""Planted mistakes for the oracle, to show that its pins catch them.

Each entry replaces one oracle function with a plausible wrong version: a
dropped term or factor, a wrong sign, root, exponent or index, a flipped tie
rule.  ``apply(name)`` installs one in both the ``oracle`` package and its
``entmax_oracle`` module (the package re-exports the module's functions, and
the oracle calls them through the module), so that the pin tests and the
oracle's own callers see it.  Used only by ``test_oracle_mutants.py``
through ``conftest.py``; never installed otherwise.
"""
import math

import numpy as np

import oracle
import oracle.entmax_oracle as M

_orig = {}


def _get(name):
    if name not in _orig:
        _orig[name] = getattr(M, name)
    return _orig[name]


def _entmax15_wrong_root(z, alpha):
    if alpha != 1.5:
        return _get("entmax_threshold")(z, alpha)
    zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    csum, csq = np.cumsum(zs), np.cumsum(zs * zs)
    tau = None
    for k in range(1, len(zs) + 1):
        mean, msq = csum[k - 1] / k, csq[k - 1] / k
        dk = 1.0 / k - (msq - mean * mean)
        if dk >= 0.0 and mean - math.sqrt(dk) <= zs[k - 1]:
            tau = mean + math.sqrt(dk)
    return tau


def _sparsemax_extra_element(z, alpha):
    if alpha != 2.0:
        return _get("entmax_threshold")(z, alpha)
    zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    csum = np.cumsum(zs)
    K = 1
    for k in range(1, len(zs) + 1):
        if 1.0 + k * zs[k - 1] > csum[k - 1]:
            K = k
    K = min(K + 1, len(zs))
    return (csum[K - 1] - 1.0) / K


def _probs_wrong_exponent(z, tau, alpha):
    return np.maximum(np.asarray(z, dtype=np.float64) - tau, 0.0) ** (alpha - 1.0)


def _scores_no_scale(q, keys, scale):
    return _get("token_scores")(q, keys, 1.0)


def _bbox_max_of_sums(q, kmin, kmax, scale):
    return scale * np.maximum(kmin @ q, kmax @ q)


def _moments_no_scale_sq(q, mean, var, scale):
    mu, s2 = _get("gauss_moments")(q, mean, var, scale)
    return mu, s2 / (scale * scale)


def _moments_q_not_squared(q, mean, var, scale):
    mu, _ = _get("gauss_moments")(q, mean, var, scale)
    return mu, scale * scale * (var @ np.abs(q))


def _sample_variance(keys):
    kmin, kmax, mean, var = _get("page_metadata")(keys)
    n = keys.shape[0]
    return kmin, kmax, mean, var * n / (n - 1) if n > 1 else var


def _topk_ties_high(g, k):
    n = len(g)
    order = sorted(range(n), key=lambda p: (-g[p], -p))
    return np.array(sorted(order[:min(k, n)]), dtype=np.int64)


def _normaliser_unweighted(tau, m, s, n_tok, r):
    return _get("gauss_normaliser")(tau, m, s, np.ones_like(np.asarray(n_tok)), r)


def _max_estimate_no_2(mu, sigma2, n_tok):
    n = np.asarray(n_tok, dtype=np.float64)
    return mu + np.sqrt(np.maximum(sigma2, 0.0)) * np.sqrt(np.log(n))


def _excess_sign_flip(m, s, tau, r):
    # Phi and phi taken at -c: the mirror image of the right tail
    m = np.asarray(m, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return _get("gauss_excess_moment")(2.0 * tau - m, s, tau, r)


def _keep_wrong_delta_sign(mu, sigma2, n_tok, tau_hat, alpha, delta):
    return _get("gauss_keep")(mu, sigma2, n_tok, tau_hat, alpha, -delta)


def _pages_to_tokens_skip_first(pages, n_tokens, P):
    out = []
    for p in sorted(int(x) for x in pages):
        out.extend(range(p * P + 1, min((p + 1) * P, n_tokens)))
    return np.array(out, dtype=np.int64)


def _counts_full_last(n_tokens, P):
    n_pages = (n_tokens + P - 1) // P
    return np.full(n_pages, P, dtype=np.int64)


def _excess_standard_order_off(c, r):
    return _get("excess_standard")(c, r + 1.0)


def _bisect_half_exponent(z, alpha, tol=1e-13):
    # the bracket search with r = alpha - 1 instead of 1 / (alpha - 1)
    return _get("entmax_threshold_bisect")(z, 1.0 + 1.0 / (alpha - 1.0), tol)


MUTANTS = {
    "entmax15_wrong_root": ("entmax_threshold", _entmax15_wrong_root),
    "sparsemax_extra_element": ("entmax_threshold", _sparsemax_extra_element),
    "probs_wrong_exponent": ("entmax_probs", _probs_wrong_exponent),
    "scores_no_scale": ("token_scores", _scores_no_scale),
    "bbox_max_of_sums": ("bbox_bound", _bbox_max_of_sums),
    "moments_no_scale_sq": ("gauss_moments", _moments_no_scale_sq),
    "moments_q_not_squared": ("gauss_moments", _moments_q_not_squared),
    "sample_variance": ("page_metadata", _sample_variance),
    "topk_ties_high": ("select_topk", _topk_ties_high),
    "normaliser_unweighted": ("gauss_normaliser", _normaliser_unweighted),
    "max_estimate_no_2": ("page_max_estimate", _max_estimate_no_2),
    "excess_sign_flip": ("gauss_excess_moment", _excess_sign_flip),
    "keep_wrong_delta_sign": ("gauss_keep", _keep_wrong_delta_sign),
    "pages_to_tokens_skip_first": ("pages_to_tokens", _pages_to_tokens_skip_first),
    "counts_full_last": ("page_token_counts", _counts_full_last),
    "excess_standard_order_off": ("excess_standard", _excess_standard_order_off),
    "bisect_reciprocal_exponent": ("entmax_threshold_bisect", _bisect_half_exponent),
}


def apply(name: str) -> None:
    target, fn = MUTANTS[name]
    _get(target)
    setattr(M, target, fn)
    setattr(oracle, target, fn)
