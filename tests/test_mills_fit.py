"""The Gaussian selector's normal tail uses a fitted rational Mills ratio
(select.hip, norm_cdf_pdf).  fit_mills.py, beside the kernel, regenerates
such a fit and checks the committed constants against
R(x) = sqrt(pi/2) erfcx(x / sqrt(2)) on [0, 14]."""
import importlib.util
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
PATH = os.path.join(HERE, "..", "sparse_entmax_attention_amd", "csrc", "fit_mills.py")


def _mod():
    spec = importlib.util.spec_from_file_location("fit_mills", PATH)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_kernel_constants_meet_their_bound():
    e64, e32, positive = _mod().check(verbose=False)
    assert e64 <= 2e-8
    assert e32 <= 1e-6
    assert positive


def test_refit_reaches_the_same_accuracy():
    num, den, err = _mod().fit(iters=80, grid=8001)
    assert err <= 2e-8
    assert all(c > 0 for c in num + den)
    assert den[-1] == pytest.approx(1.0)
