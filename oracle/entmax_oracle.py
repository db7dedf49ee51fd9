"""fp64 reference implementation of the EntmaxKV support-aware decode step.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the library.

Sources.  Three web pages describe the method: the English "Technical
Summary: EntmaxKV - Support-Aware Decoding for Entmax Attention"
(gist.science), its Chinese translation (gist.science/zh) and the arXiv
abstract of "EntmaxKV: Support-Aware Decoding for Entmax Attention"
(mlsanity.com index page).  They fix the pipeline (page scoring, candidate
selection, sparse entmax attention), the two page summaries (coordinate-wise
key box; per-coordinate key mean and variance), the two selectors (top-k by
box bound; Gaussian estimate of the entmax threshold with a margin Delta)
and the two guarantees (error at most 2 B delta; exactness when the kept set
covers the support).  They print no formulas beyond symbol names, no worked
numbers and no code.  Every formula below is the plainest reading of those
passages; the readings are listed where each function is defined.

Conventions.  Scores s_i = scale * <q, k_i>.  Entmax works on
z_i = (alpha - 1) s_i with threshold tau and exponent r = 1/(alpha - 1):
p_i = max(z_i - tau, 0)^r with sum_i p_i = 1.  alpha = 2 is sparsemax,
alpha = 1.5 is 1.5-entmax.

Pinning (see tests/test_oracle_*.py):
  * entmax_threshold / entmax_probs: pinned (brute-force support
    enumeration, bisection vs sort closed forms, invariants, two-point
    closed forms, hand-derived fixtures).
  * page_metadata: pinned (identities and special cases).
  * bbox_bound: pinned (bound invariant, one-token pages, sign-split form).
  * gauss_moments: pinned (exact variance of the score of a page's tokens
    in the single-coordinate case; Monte Carlo).
  * select_topk: pinned (brute force over subsets, nesting, k >= n).
  * group_bound: pinned (on one-token pages the group value is the largest
    exact token score over the query heads; on any page it bounds every
    head's token scores and is attained by one head's bound).
  * gauss_excess_moment, excess_standard: pinned (numerical quadrature of
    the defining integral for r in {1, 2, 4/3, 3, 4, 7.5} on both sides of
    the series switch, the closed forms at r = 1 and 2, the recurrence
    J_r = (r-1) J_(r-2) - c J_(r-1), Monte Carlo).
  * solve_tau_hat: pinned (zero-variance limit equals the exact entmax
    threshold of the repeated means; monotonicity; uniqueness).
  * page_max_estimate: pinned by the defining property of the classical
    bound it reads the 'estimated maximum score' as (at least the Monte
    Carlo expected maximum of n draws, exact at n = 1, within 35 % above the
    mean at n = 16 and 64).
  * gauss_keep: parity unpinned beyond self-consistency.  The comparison
    (alpha - 1) * estimate > tau_hat - delta in z units is a reading of the
    summary's Gaussian selector paragraph; no page fixes it numerically.
    Limits (Delta -> inf keeps every page) are pinned.
  * bf16_bits_to_f64, unit_tokens: pinned (exact decoding of known bit
    patterns; a scatter of numbered tokens through a random page table
    gathers back in order).
  Planted mistakes in these functions (tests/oracle_mutants.py: dropped
  factors, wrong signs, roots, exponents, indices and tie rules) each fail
  at least one pin (tests/test_oracle_mutants.py).
  * softmax_attend: pinned (shift invariance, alpha -> 1 limit of entmax).
  * dropped_mass, softmax_dropped_mass, support_recall,
    matched_budget_quality: pinned (covering sets give zero dropped mass,
    full recall and the full-cache output; the softmax mass outside a set
    equals 1 - exp(lse(kept) - lse(all)); the output error stays within
    2 B delta).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special as _sp

__all__ = [
    "bf16_bits_to_f64", "unit_tokens", "page_token_counts", "page_metadata",
    "unit_metadata", "token_scores", "bbox_bound", "gauss_moments",
    "group_bound", "select_topk", "excess_standard", "gauss_excess_moment",
    "gauss_normaliser", "solve_tau_hat",
    "page_max_estimate", "gauss_keep", "entmax_threshold",
    "entmax_threshold_bisect", "entmax_probs", "entmax_attend",
    "softmax_attend", "pages_to_tokens", "decode_unit", "dropped_mass",
    "softmax_dropped_mass", "support_recall", "matched_budget_quality",
]


# ---------------------------------------------------------------------------
# Input decoding and the paged layout
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of raw bfloat16 bit patterns (uint16 array).

    A bfloat16 is the top half of an IEEE binary32, so shifting its 16 bits
    into the high half of a 32-bit word gives the float32 with the same
    value, which widens to fp64 without rounding.
    """
    w = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)
    return w.view(np.float32).astype(np.float64)


def unit_tokens(pool: np.ndarray, page_table_row: np.ndarray, kv_head: int,
                n_tokens: int) -> np.ndarray:
    """Rows [n_tokens][D] of one (sequence, KV head) in logical order.

    Gathers through the page table: logical token i lives in page i // P at
    physical slot page_table_row[i // P], offset i % P
    [Technical Summary, §2 (paged pipeline) and §2.C (load only the chosen
    pages)].  ``pool`` is [num_slots][H_kv][P][D] in fp64.
    """
    P = pool.shape[2]
    rows = np.empty((n_tokens, pool.shape[3]), dtype=np.float64)
    for i in range(n_tokens):
        rows[i] = pool[page_table_row[i // P], kv_head, i % P]
    return rows


def page_token_counts(n_tokens: int, P: int) -> np.ndarray:
    """Valid tokens n_p of every logical page (P, except a short last page)."""
    n_pages = (n_tokens + P - 1) // P
    return np.array([min(P, n_tokens - p * P) for p in range(n_pages)],
                    dtype=np.int64)


def pages_to_tokens(pages, n_tokens: int, P: int) -> np.ndarray:
    """Logical token indices of the given pages, ascending page order."""
    out = []
    for p in sorted(int(x) for x in pages):
        out.extend(range(p * P, min((p + 1) * P, n_tokens)))
    return np.array(out, dtype=np.int64)


# ---------------------------------------------------------------------------
# Page metadata  [Technical Summary, §2.A: box bounds and Gaussian statistics]
# ---------------------------------------------------------------------------

def page_metadata(keys: np.ndarray):
    """(kmin, kmax, mean, var) of one page's keys [n_p][D].

    The box is the coordinate-wise minimum and maximum of the page's keys;
    the Gaussian summary is the coordinate-wise first and second moments.
    Reading: the variance is the population one (divide by n_p), taken
    about the mean in a second pass; coordinates are independent (diagonal).
    """
    n = keys.shape[0]
    kmin = keys.min(axis=0)
    kmax = keys.max(axis=0)
    mean = keys.sum(axis=0) / n
    dev = keys - mean
    var = (dev * dev).sum(axis=0) / n
    return kmin, kmax, mean, var


def unit_metadata(keys: np.ndarray, P: int):
    """Per-page metadata of a token sequence [N][D]; arrays are [n_pages][D]."""
    counts = page_token_counts(keys.shape[0], P)
    out = [np.empty((len(counts), keys.shape[1])) for _ in range(4)]
    for p in range(len(counts)):
        m = page_metadata(keys[p * P:p * P + counts[p]])
        for a, x in zip(out, m):
            a[p] = x
    return tuple(out)


# ---------------------------------------------------------------------------
# Query-aware page scoring  [Technical Summary, §2.A]
# ---------------------------------------------------------------------------

def token_scores(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s_i = scale * <q, k_i> for every row of keys [N][D].

    Each row's sum is formed from that row alone (no matrix-vector kernel
    whose rounding depends on the other rows), so a token's score is the
    same whichever set of tokens it is computed with.
    """
    out = np.empty(keys.shape[0])
    for r0 in range(0, keys.shape[0], 65536):
        blk = keys[r0:r0 + 65536]
        out[r0:r0 + blk.shape[0]] = (blk * q[None, :]).sum(axis=1)
    return scale * out


def bbox_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray,
               scale: float) -> np.ndarray:
    """Box upper bound of the score of any key in each page.

    For every coordinate the product q_d * k_d over k_d in [kmin_d, kmax_d]
    is largest at one of the two ends, so scale * sum_d max(q_d kmin_d,
    q_d kmax_d) bounds every token score of the page from above.
    kmin, kmax: [n_pages][D].
    """
    lo = kmin * q[None, :]
    hi = kmax * q[None, :]
    return scale * np.maximum(lo, hi).sum(axis=1)


def gauss_moments(q: np.ndarray, mean: np.ndarray, var: np.ndarray,
                  scale: float):
    """Mean and variance of the score of a page's key under the page Gaussian.

    With independent coordinates of means mean_d and variances var_d, the
    score scale * <q, k> has mean scale * <q, mean> and variance
    scale^2 * sum_d q_d^2 var_d.  Returns (mu [n_pages], sigma2 [n_pages]).
    """
    mu = scale * (mean @ q)
    sigma2 = scale * scale * (var @ (q * q))
    return mu, sigma2


# ---------------------------------------------------------------------------
# Top-k page selection  [Technical Summary, §2.B.1]
# ---------------------------------------------------------------------------

def group_bound(ub: np.ndarray) -> np.ndarray:
    """Ranking value of every page for a KV head's G query heads.

    ub: [G][n_pages], each row one query head's box bound.  Reading: one
    selection serves all query heads of a KV head, so a page is ranked by a
    value that bounds the score of any of its tokens for any of those heads;
    the tightest such value built from the per-head bounds is their largest,
    g_p = max_h ub[h, p].
    """
    return np.asarray(ub, dtype=np.float64).max(axis=0)


def select_topk(g: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) pages with the largest bound g, returned ascending.

    Reading: equal bounds are ordered by page index (lower index first),
    and one selection serves all query heads of a KV head, ranked by the
    largest of their bounds (the caller passes that maximum as ``g``).
    """
    n = len(g)
    order = sorted(range(n), key=lambda p: (-g[p], p))
    return np.array(sorted(order[:min(k, n)]), dtype=np.int64)


# ---------------------------------------------------------------------------
# Gaussian-aware entmax selection  [Technical Summary, §2.B.2]
# ---------------------------------------------------------------------------

def _phi(c):
    return np.exp(-0.5 * c * c) / math.sqrt(2.0 * math.pi)


def _Phi(c):
    return 0.5 * _sp.erfc(-c / math.sqrt(2.0))


def excess_standard(c, r: float):
    """J_r(c) = E[max(X - c, 0)^r] for X standard normal and real r >= 1.

    J_r(c) = int_0^inf y^r phi(y + c) dy = phi(c) int_0^inf y^r e^(-c y - y^2/2) dy,
    and the last integral is Gamma(r + 1) e^(c^2/4) D_(-r-1)(c) with D the
    parabolic cylinder function (its standard integral representation), so
    J_r(c) = Gamma(r + 1) e^(-c^2/4) D_(-r-1)(c) / sqrt(2 pi).  Far below the
    mean (c < -30), where D overflows in double, X - c = a (1 + X/a) with
    a = -c and the expectation is the series sum_k C(r, 2k) (2k-1)!! a^(r-2k)
    (odd moments vanish; the mass where 1 + X/a < 0 is below 1e-190).
    """
    c = np.asarray(c, dtype=np.float64)
    out = np.empty(c.shape)
    far = c < -30.0
    near = ~far
    if np.any(near):
        d, _ = _sp.pbdv(-r - 1.0, c[near])
        out[near] = (_sp.gamma(r + 1.0) * np.exp(-0.25 * c[near] ** 2) * d
                     / math.sqrt(2.0 * math.pi))
    if np.any(far):
        a = -c[far]
        tot = np.ones(a.shape)
        dfact = 1.0
        for k in range(1, 16):
            dfact *= 2 * k - 1
            tot += _sp.binom(r, 2 * k) * dfact * a ** (-2.0 * k)
        out[far] = a ** r * tot
    return out


def gauss_excess_moment(m, s, tau, r: float):
    """E[max(Z - tau, 0)^r] for Z ~ N(m, s^2), real r >= 1.

    Writing Z - tau = u + s X with u = m - tau and X standard normal, the
    positive part is non-zero for X > -u/s; integrating against the normal
    density gives, with c = u/s,
      r = 1:  u Phi(c) + s phi(c)
      r = 2:  (u^2 + s^2) Phi(c) + u s phi(c)
    otherwise s^r J_r(-c) (excess_standard), and max(u, 0)^r when s = 0.
    """
    m = np.asarray(m, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    u = m - tau
    out = np.empty(np.broadcast(u, s).shape)
    u, s = np.broadcast_arrays(u, s)
    zero = s <= 0.0
    pos = ~zero
    if np.any(zero):
        out[zero] = np.maximum(u[zero], 0.0) ** r
    if np.any(pos):
        uu, ss = u[pos], s[pos]
        c = uu / ss
        if r == 1:
            out[pos] = uu * _Phi(c) + ss * _phi(c)
        elif r == 2:
            out[pos] = (uu * uu + ss * ss) * _Phi(c) + uu * ss * _phi(c)
        else:
            out[pos] = ss ** r * excess_standard(-c, r)
    return out


def gauss_normaliser(tau: float, m, s, n_tok, r: int) -> float:
    """F(tau) = sum_p n_p E[max(Z_p - tau, 0)^r].

    Reading of the 'approximate normalization equation': every token of page
    p is treated as an independent draw of the page's score Gaussian
    Z_p ~ N((alpha-1) mu_p, (alpha-1)^2 sigma_p^2), so the expected entmax
    mass at threshold tau is F(tau); the selector's threshold solves F = 1.
    """
    return float(np.sum(np.asarray(n_tok, dtype=np.float64)
                        * gauss_excess_moment(m, s, tau, r)))


def solve_tau_hat(mu: np.ndarray, sigma2: np.ndarray, n_tok: np.ndarray,
                  alpha: float, tol: float = 1e-12) -> float:
    """Estimated entmax threshold from page Gaussians, by bisection.

    F is continuous and strictly decreasing where positive.  At
    tau_lo = max_p m_p - 1 Jensen's inequality gives F >= n_p* >= 1; the
    upper end doubles its distance from tau_lo until F <= 1.
    """
    r = _gauss_exponent(alpha)
    m = (alpha - 1.0) * np.asarray(mu, dtype=np.float64)
    s = (alpha - 1.0) * np.sqrt(np.maximum(np.asarray(sigma2, np.float64), 0))
    lo = float(np.max(m)) - 1.0
    step = 1.0
    hi = lo + step
    while gauss_normaliser(hi, m, s, n_tok, r) > 1.0:
        step *= 2.0
        hi = lo + step
    while hi - lo > tol:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if gauss_normaliser(mid, m, s, n_tok, r) >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def page_max_estimate(mu: np.ndarray, sigma2: np.ndarray,
                      n_tok: np.ndarray) -> np.ndarray:
    """Estimated largest score among a page's n_p tokens: mu + sigma sqrt(2 ln n_p).

    Reading of the 'estimated maximum score': the classical upper bound on
    the expected maximum of n Gaussians of standard deviation sigma.
    """
    n = np.asarray(n_tok, dtype=np.float64)
    return mu + np.sqrt(np.maximum(sigma2, 0.0)) * np.sqrt(2.0 * np.log(n))


def gauss_keep(mu: np.ndarray, sigma2: np.ndarray, n_tok: np.ndarray,
               tau_hat: np.ndarray, alpha: float, delta: float) -> np.ndarray:
    """Pages kept by the Gaussian selector for one KV head, ascending.

    mu, sigma2: [G][n_pages] for the KV head's G query heads; tau_hat: [G].
    Page p is kept when some query head h has
    (alpha-1) * mhat_{h,p} > tau_hat_h - delta (strict; delta in z units).
    Reading for the empty case, which the pages leave open: keep the one page
    maximising max_h [(alpha-1) mhat_{h,p} - tau_hat_h], lower index on ties.
    """
    G, n = mu.shape
    zhat = np.stack([(alpha - 1.0) * page_max_estimate(mu[h], sigma2[h], n_tok)
                     for h in range(G)])
    kept = [p for p in range(n)
            if any(zhat[h, p] > tau_hat[h] - delta for h in range(G))]
    if not kept:
        gap = np.max(zhat - np.asarray(tau_hat)[:, None], axis=0)
        best = max(range(n), key=lambda p: (gap[p], -p))
        kept = [best]
    return np.array(kept, dtype=np.int64)


# ---------------------------------------------------------------------------
# alpha-entmax  [Technical Summary, §2 and §2.C; arXiv abstract]
# ---------------------------------------------------------------------------

def _gauss_exponent(alpha: float) -> float:
    """r = 1/(alpha - 1) for the Gaussian selector, which needs r >= 1
    (alpha <= 2): then x -> max(x - tau, 0)^r is convex and the Jensen bound
    and the monotone Newton iteration below hold.  Exactly 1 or 2 for
    alpha = 2 or 1.5, so that the closed forms apply."""
    if not (1.0 < alpha <= 2.0):
        raise ValueError("the Gaussian selector needs 1 < alpha <= 2")
    r = 1.0 / (alpha - 1.0)
    return float(round(r)) if abs(r - round(r)) < 1e-12 else r


def _integer_exponent(alpha: float) -> int:
    r = 1.0 / (alpha - 1.0)
    if abs(r - round(r)) > 1e-12 or round(r) not in (1, 2):
        raise ValueError("closed forms exist for alpha in {1.5, 2} only")
    return int(round(r))


def entmax_threshold(z: np.ndarray, alpha: float) -> float:
    """tau with sum_i max(z_i - tau, 0)^(1/(alpha-1)) = 1, exactly.

    alpha = 2 (sparsemax): sort z descending with prefix sums c_k; the
    support size K is the largest k with 1 + k z_(k) > c_k and
    tau = (c_K - 1)/K.
    alpha = 1.5: for a support made of the k largest entries, the squares
    sum to one when (mean_k - tau)^2 = 1/k - (meansq_k - mean_k^2); with
    delta_k that right-hand side and tau_k = mean_k - sqrt(delta_k), the
    support size K is the largest k with delta_k >= 0 and tau_k <= z_(k).
    Other alpha: bisection (entmax_threshold_bisect).
    """
    if alpha == 2.0:
        zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
        csum = np.cumsum(zs)
        K = 1
        for k in range(1, len(zs) + 1):
            if 1.0 + k * zs[k - 1] > csum[k - 1]:
                K = k
        return (csum[K - 1] - 1.0) / K
    if alpha == 1.5:
        zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
        csum = np.cumsum(zs)
        csq = np.cumsum(zs * zs)
        tau = None
        for k in range(1, len(zs) + 1):
            mean = csum[k - 1] / k
            msq = csq[k - 1] / k
            dk = 1.0 / k - (msq - mean * mean)
            if dk < 0.0:
                continue
            tk = mean - math.sqrt(dk)
            if tk <= zs[k - 1]:
                tau = tk
        return tau
    return entmax_threshold_bisect(z, alpha)


def entmax_threshold_bisect(z: np.ndarray, alpha: float,
                            tol: float = 1e-13) -> float:
    """tau by bisection on [max z - 1, max z - n^-(alpha-1)].

    At the left end the largest entry alone contributes 1; at the right end
    every entry contributes at most 1/n.  The mass is decreasing in tau.
    """
    z = np.asarray(z, dtype=np.float64)
    r = 1.0 / (alpha - 1.0)
    zmax = float(np.max(z))
    lo = zmax - 1.0
    hi = zmax - len(z) ** (-(alpha - 1.0))
    while hi - lo > tol:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if np.sum(np.maximum(z - mid, 0.0) ** r) >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def entmax_probs(z: np.ndarray, tau: float, alpha: float) -> np.ndarray:
    """p_i = max(z_i - tau, 0)^(1/(alpha-1))."""
    r = 1.0 / (alpha - 1.0)
    return np.maximum(np.asarray(z, dtype=np.float64) - tau, 0.0) ** r


def entmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                  scale: float, alpha: float):
    """alpha-entmax attention of one query over rows keys/vals [N][D].

    Returns (o [D], tau, p [N]); o = sum_i p_i v_i summed in row order.
    """
    z = (alpha - 1.0) * token_scores(q, keys, scale)
    tau = entmax_threshold(z, alpha)
    p = entmax_probs(z, tau, alpha)
    o = np.zeros(vals.shape[1])
    for i in range(len(p)):
        if p[i] != 0.0:
            o += p[i] * vals[i]
    return o, tau, p


def softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                   scale: float):
    """Softmax attention of one query: (o [D], log-sum-exp of the scores).

    Uses the max-shifted exponentials, which leave the weights unchanged.
    """
    s = token_scores(q, keys, scale)
    m = float(np.max(s))
    w = np.exp(s - m)
    tot = float(np.sum(w))
    o = (w / tot) @ vals
    return o, m + math.log(tot)


# ---------------------------------------------------------------------------
# One (sequence, KV head) decode step  [Technical Summary, §2 A-C]
# ---------------------------------------------------------------------------

def decode_unit(qs: np.ndarray, keys: np.ndarray, vals: np.ndarray, P: int,
                scale: float, alpha: float, selector: str, k: int = 0,
                delta: float = 0.0, pages=None) -> dict:
    """Full decode step of one KV head's G query heads.

    qs: [G][D]; keys, vals: [N][D] in logical order.  ``selector`` is
    "topk" (box bound, largest over the group, top k), "gauss" (Gaussian
    threshold estimate per query head, union over the group), "full" (every
    page) or "given" (``pages`` supplied, e.g. another implementation's
    selection, to check its attention output on that very set).
    Returns a dict with the selection, per-head tau, outputs and the page
    scores that drove the selection.
    """
    G = qs.shape[0]
    N = keys.shape[0]
    counts = page_token_counts(N, P)
    res = {}
    if selector in ("topk", "gauss"):
        kmin, kmax, mean, var = unit_metadata(keys, P)
    if selector == "topk":
        ub = np.stack([bbox_bound(qs[h], kmin, kmax, scale) for h in range(G)])
        g = group_bound(ub)
        sel = select_topk(g, k)
        res.update(ub=ub, g=g)
    elif selector == "gauss":
        mus, sig2s = zip(*[gauss_moments(qs[h], mean, var, scale)
                           for h in range(G)])
        mu, sig2 = np.stack(mus), np.stack(sig2s)
        tau_hat = np.array([solve_tau_hat(mu[h], sig2[h], counts, alpha)
                            for h in range(G)])
        sel = gauss_keep(mu, sig2, counts, tau_hat, alpha, delta)
        res.update(mu=mu, sigma2=sig2, tau_hat=tau_hat)
    elif selector == "full":
        sel = np.arange(len(counts), dtype=np.int64)
    elif selector == "given":
        sel = np.array(sorted(int(x) for x in pages), dtype=np.int64)
    else:
        raise ValueError(selector)
    toks = pages_to_tokens(sel, N, P)
    outs, taus = [], []
    for h in range(G):
        o, tau, _ = entmax_attend(qs[h], keys[toks], vals[toks], scale, alpha)
        outs.append(o)
        taus.append(tau)
    res.update(sel=sel, tokens=toks, out=np.stack(outs), tau=np.array(taus))
    return res


def dropped_mass(q: np.ndarray, keys: np.ndarray, kept_tokens, scale: float,
                 alpha: float):
    """Full-cache entmax mass of the tokens outside a kept set.

    Returns (delta, p_full, tau_full) for one query: delta is the mass the
    full-cache distribution puts on dropped tokens, the quantity that bounds
    the output error by 2 B delta, B bounding the value norms
    [Technical Summary, §3].
    """
    z = (alpha - 1.0) * token_scores(q, keys, scale)
    tau = entmax_threshold(z, alpha)
    p = entmax_probs(z, tau, alpha)
    mask = np.ones(len(z), dtype=bool)
    mask[np.asarray(kept_tokens, dtype=np.int64)] = False
    return float(p[mask].sum()), p, tau


def softmax_dropped_mass(q: np.ndarray, keys: np.ndarray, kept_tokens,
                         scale: float) -> float:
    """Full-cache softmax mass of the tokens outside a kept set, summed
    directly from the normalised weights (softmax gives every token weight,
    so this is zero only when every token is kept)."""
    s = token_scores(q, keys, scale)
    w = np.exp(s - np.max(s))
    w /= np.sum(w)
    mask = np.ones(len(s), dtype=bool)
    mask[np.asarray(kept_tokens, dtype=np.int64)] = False
    return float(w[mask].sum())


def support_recall(p_full: np.ndarray, kept_tokens) -> float:
    """Share of the full-cache entmax support (p_i > 0) inside a kept set."""
    support = np.flatnonzero(np.asarray(p_full) > 0.0)
    kept = np.zeros(len(p_full), dtype=bool)
    kept[np.asarray(kept_tokens, dtype=np.int64)] = True
    return float(kept[support].sum()) / max(len(support), 1)


def matched_budget_quality(qs: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                           P: int, scale: float, alpha: float, pages) -> dict:
    """Entmax against softmax on one kept page set (the same budget for both).

    Per query head of qs [G][D]: the full-cache mass each distribution puts
    outside the kept tokens (delta_entmax, delta_softmax), the share of the
    entmax support inside them (recall), and the relative L2 error of the
    output computed on the kept tokens alone against the full-cache output
    (err_entmax, err_softmax).  The Technical Summary (§3) bounds the entmax
    error by 2 B delta and notes that it vanishes when the kept set covers
    the support; softmax weights never vanish, so its mass outside any
    proper subset is positive.
    """
    N = keys.shape[0]
    toks = pages_to_tokens(pages, N, P)
    out = {k: [] for k in ("delta_entmax", "delta_softmax", "recall",
                           "err_entmax", "err_softmax")}
    for q in qs:
        de, p_full, _ = dropped_mass(q, keys, toks, scale, alpha)
        o_full = p_full @ vals
        o_kept, _, _ = entmax_attend(q, keys[toks], vals[toks], scale, alpha)
        so_full, _ = softmax_attend(q, keys, vals, scale)
        so_kept, _ = softmax_attend(q, keys[toks], vals[toks], scale)
        out["delta_entmax"].append(de)
        out["delta_softmax"].append(softmax_dropped_mass(q, keys, toks, scale))
        out["recall"].append(support_recall(p_full, toks))
        out["err_entmax"].append(float(np.linalg.norm(o_kept - o_full) /
                                       np.linalg.norm(o_full)))
        out["err_softmax"].append(float(np.linalg.norm(so_kept - so_full) /
                                        np.linalg.norm(so_full)))
    return {k: np.array(v) for k, v in out.items()}
