#!/usr/bin/env python3
"""Fit and check the rational Mills-ratio approximation of select.hip.

select.hip evaluates the upper normal tail as Q(a) = phi(a) R(a), a >= 0,
with the Mills ratio R(x) = Q(x) / phi(x) = sqrt(pi/2) erfcx(x / sqrt(2))
replaced by num(x) / den(x): num of degree 4, den of degree 5 with den(0) =
1, all coefficients positive (so both are increasing on x >= 0, with no
pole, and R ~ n4 / (d5 x) ~ 1/x for large x when n4 = d5).

    python fit_mills.py          # refit on [0, 14] and report both fits
    python fit_mills.py --check  # only check the constants in select.hip

The fit minimises the largest relative error over a dense grid by Lawson's
iteratively reweighted least squares on the linearised residual
num(x) - R(x) den(x) (weights grow where the relative error is largest),
from an unweighted least-squares start.  Minimax fits of this kind have
many nearly equal optima, so a refit need not reproduce the committed
digits; what matters, and what the check asserts, is the error of the
constants the kernel uses: at most 2e-8 relative in double on [0, 14], and
at most 1e-6 relative when the kernel's float32 Horner evaluation is
emulated with numpy float32.
"""
from __future__ import annotations

import argparse
import os
import re
import sys

import numpy as np
from scipy.special import erfcx

HERE = os.path.dirname(os.path.abspath(__file__))
X_MAX = 14.0


def mills(x):
    return np.sqrt(np.pi / 2.0) * erfcx(np.asarray(x, dtype=np.float64) / np.sqrt(2.0))


def kernel_constants(path=os.path.join(HERE, "select.hip")):
    """(num, den) coefficients as written in norm_cdf_pdf, highest degree
    first (the order of the Horner steps)."""
    src = open(path).read()
    body = src[src.index("void norm_cdf_pdf"):]
    body = body[:body.index("}")]
    num = [float(v) for v in re.findall(r"float num = ([0-9.e+-]+)f;", body)]
    num += [float(v) for v in re.findall(r"num = fmaf\(num, a, ([0-9.e+-]+)f\);", body)]
    den = [float(v) for v in re.findall(r"float den = ([0-9.e+-]+)f;", body)]
    den += [float(v) for v in re.findall(r"den = fmaf\(den, a, ([0-9.e+-]+)f\);", body)]
    if len(num) != 5 or len(den) != 6:
        raise RuntimeError("unexpected form of norm_cdf_pdf in %s" % path)
    return num, den


def rel_error(num, den, x, dtype=np.float64):
    """Relative error of num(x)/den(x) against R(x); Horner in `dtype` with
    fused multiply-adds emulated by rounding after each step (float32: a
    product and a sum each rounded, a slightly pessimistic model of fmaf)."""
    xs = x.astype(dtype)
    n = np.full_like(xs, dtype(num[0]))
    for c in num[1:]:
        n = (n * xs + dtype(c)).astype(dtype)
    d = np.full_like(xs, dtype(den[0]))
    for c in den[1:]:
        d = (d * xs + dtype(c)).astype(dtype)
    r = (n / d).astype(np.float64)
    ref = mills(x)
    return np.abs(r / ref - 1.0)


def fit(deg_num=4, deg_den=5, iters=200, grid=20001):
    """Lawson fit; returns (num, den) highest degree first, den(0) = 1."""
    x = np.linspace(0.0, X_MAX, grid)
    R = mills(x)
    # unknowns: num coefficients n0..n4, den coefficients d1..d5 (d0 = 1);
    # residual over R: (num - R den) / R = 0
    cols = [x ** k / R for k in range(deg_num + 1)]
    cols += [-(x ** k) for k in range(1, deg_den + 1)]
    A = np.stack(cols, axis=1)
    b = np.ones_like(x)
    w = np.ones_like(x) / len(x)
    best = None
    for _ in range(iters):
        sw = np.sqrt(w)
        coef, *_ = np.linalg.lstsq(A * sw[:, None], b * sw, rcond=None)
        num = coef[:deg_num + 1][::-1]
        den = np.concatenate([coef[deg_num + 1:][::-1], [1.0]])
        err = rel_error(num, den, x)
        if best is None or err.max() < best[0]:
            best = (err.max(), num, den)
        w = w * (err + 1e-300)
        w /= w.sum()
    return best[1].tolist(), best[2].tolist(), best[0]


def check(verbose=True):
    num, den = kernel_constants()
    x = np.linspace(0.0, X_MAX, 200001)
    e64 = rel_error(num, den, x).max()
    e32 = rel_error(num, den, x, np.float32).max()
    positive = all(c > 0 for c in num + den)
    if verbose:
        print("select.hip constants: max relative error %.3g (double), "
              "%.3g (float32 Horner), all positive: %s" % (e64, e32, positive))
    return e64, e32, positive


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true")
    args = ap.parse_args()
    e64, e32, positive = check()
    ok = e64 <= 2e-8 and e32 <= 1e-6 and positive
    if not args.check:
        num, den, err = fit()
        print("refit on [0, %g]: max relative error %.3g" % (X_MAX, err))
        print("  num (x^4 .. x^0):", " ".join("%.9e" % c for c in num))
        print("  den (x^5 .. x^0):", " ".join("%.9e" % c for c in den))
        print("  all positive:", all(c > 0 for c in num + den))
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
