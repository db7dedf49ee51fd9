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


def _bf16_wrong_shift(bits):
    w = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15)
    return w.view(np.float32).astype(np.float64)


def _unit_tokens_offset_order(pool, page_table_row, kv_head, n_tokens):
    # rows of each page taken in reverse
    P = pool.shape[2]
    rows = _get("unit_tokens")(pool, page_table_row, kv_head, n_tokens)
    out = rows.copy()
    for p0 in range(0, n_tokens, P):
        p1 = min(p0 + P, n_tokens)
        out[p0:p1] = rows[p0:p1][::-1]
    return out


def _softmax_lse_unshifted(q, keys, vals, scale):
    o, lse = _get("softmax_attend")(q, keys, vals, scale)
    s = _get("token_scores")(q, keys, scale)
    return o, lse - float(np.max(s))


def _entmax_attend_unnormalised_tau(q, keys, vals, scale, alpha):
    # threshold taken on the scores instead of z = (alpha - 1) s
    s = _get("token_scores")(q, keys, scale)
    tau = M.entmax_threshold(s, alpha)
    p = M.entmax_probs(s, tau, alpha)
    return p @ vals, tau, p


def _dropped_mass_of_kept(q, keys, kept_tokens, scale, alpha):
    d, p, tau = _get("dropped_mass")(q, keys, kept_tokens, scale, alpha)
    return 1.0 - d, p, tau


def _softmax_dropped_unnormalised(q, keys, kept_tokens, scale):
    s = M.token_scores(q, keys, scale)
    w = np.exp(s - np.max(s))
    mask = np.ones(len(s), dtype=bool)
    mask[np.asarray(kept_tokens, dtype=np.int64)] = False
    return float(w[mask].sum())


def _recall_over_kept(p_full, kept_tokens):
    support = np.flatnonzero(np.asarray(p_full) > 0.0)
    kept = np.zeros(len(p_full), dtype=bool)
    kept[np.asarray(kept_tokens, dtype=np.int64)] = True
    return float(kept[support].sum()) / max(int(kept.sum()), 1)


def _keep_fallback_smallest_gap(mu, sigma2, n_tok, tau_hat, alpha, delta):
    kept = _get("gauss_keep")(mu, sigma2, n_tok, tau_hat, alpha, delta)
    if len(kept) != 1:
        return kept
    G, n = mu.shape
    zhat = np.stack([(alpha - 1.0) * M.page_max_estimate(mu[h], sigma2[h], n_tok)
                     for h in range(G)])
    if any(zhat[h, kept[0]] > tau_hat[h] - delta for h in range(G)):
        return kept
    gap = np.max(zhat - np.asarray(tau_hat)[:, None], axis=0)
    return np.array([int(np.argmin(gap))], dtype=np.int64)


def _keep_first_head_only(mu, sigma2, n_tok, tau_hat, alpha, delta):
    return _get("gauss_keep")(mu[:1], sigma2[:1], n_tok, tau_hat[:1], alpha, delta)


def _group_bound_head0(ub):
    return np.asarray(ub, dtype=np.float64)[0].copy()


def _group_bound_mean(ub):
    return np.asarray(ub, dtype=np.float64).mean(axis=0)


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
    "bf16_wrong_shift": ("bf16_bits_to_f64", _bf16_wrong_shift),
    "unit_tokens_rows_reversed": ("unit_tokens", _unit_tokens_offset_order),
    "softmax_lse_unshifted": ("softmax_attend", _softmax_lse_unshifted),
    "entmax_attend_on_scores": ("entmax_attend", _entmax_attend_unnormalised_tau),
    "dropped_mass_of_kept": ("dropped_mass", _dropped_mass_of_kept),
    "softmax_dropped_unnormalised": ("softmax_dropped_mass", _softmax_dropped_unnormalised),
    "recall_over_kept": ("support_recall", _recall_over_kept),
    "keep_fallback_smallest_gap": ("gauss_keep", _keep_fallback_smallest_gap),
    "keep_first_head_only": ("gauss_keep", _keep_first_head_only),
    "group_bound_head0": ("group_bound", _group_bound_head0),
    "group_bound_mean": ("group_bound", _group_bound_mean),
}


def apply(name: str) -> None:
    target, fn = MUTANTS[name]
    _get(target)
    setattr(M, target, fn)
    setattr(oracle, target, fn)
