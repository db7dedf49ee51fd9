"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function the header declares, and
reject invalid arguments on the host before anything is launched.  The
pointers handed in below are never dereferenced by the host code (only
checked for NULL and alignment), and every call here fails validation, so
no device work is ever started.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_entmax_attention_amd import _binding as B

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "entmaxkv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ekv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGNATURES)


def test_version_and_status_strings(lib):
    assert B.ekv_version() == 10000
    for code, name in [(0, "EKV_OK"), (1, "EKV_ERR_INVALID_ARG"),
                       (2, "EKV_ERR_UNSUPPORTED"), (3, "EKV_ERR_WORKSPACE"),
                       (4, "EKV_ERR_HIP")]:
        assert lib.ekv_status_string(code).decode() == name


FAKE = 0x100000  # 1 MiB: 256-byte aligned, never dereferenced on the host


def _kv(**kw):
    d = dict(batch=1, num_kv_heads=8, group=4, head_dim=128, page_size=32,
             num_slots=1024, max_pages=1024, kv_dtype=B.EKV_BF16, k=FAKE,
             v=FAKE, page_table=FAKE, seq_lens=FAKE)
    d.update(kw)
    return B.ekv_paged_kv(**d)


def test_workspace_sizes(lib):
    kv = _kv()
    units, G, D, cap = 8, 4, 128, 1024 * 32
    mc = (1024 + 15) // 16
    dec = lib.ekv_workspace_size(B.EKV_OP_ENTMAX_DECODE, ctypes.byref(kv), 0)
    assert dec >= units * G * cap * 4 + units * mc * G * D * 4
    assert dec % 256 == 0
    topk = lib.ekv_workspace_size(B.EKV_OP_SELECT_TOPK, ctypes.byref(kv), 16)
    assert topk >= units * 1024 * 4
    gauss = lib.ekv_workspace_size(B.EKV_OP_SELECT_GAUSS, ctypes.byref(kv), 0)
    assert gauss == units * G * ((1024 + 63) // 64) * 8  # page mask per head and tile
    assert lib.ekv_workspace_size(99, ctypes.byref(kv), 0) == 0
    # small-selection decode: 256 bytes of arrival counters (8 units), then
    # the scores of max_count pages for every query head
    small = lib.ekv_workspace_size(B.EKV_OP_ENTMAX_DECODE_SMALL, ctypes.byref(kv), 16)
    assert small == 256 + units * G * 16 * 32 * 4
    assert lib.ekv_workspace_size(B.EKV_OP_ENTMAX_DECODE_SMALL, ctypes.byref(kv), 0) == 0
    # score buffers: per-page values plus 64-page tile summaries
    T = (1024 + 63) // 64
    assert lib.ekv_score_size(ctypes.byref(kv), B.EKV_SCORE_BBOX) == 32 * 1024 + 8 * T
    assert lib.ekv_score_size(ctypes.byref(kv), B.EKV_SCORE_GAUSS) == 32 * 1024 * 2 + 32 * T * 4
    odd = _kv(num_kv_heads=1, group=1, max_pages=5)  # tile rows start 4-aligned
    assert lib.ekv_score_size(ctypes.byref(odd), B.EKV_SCORE_GAUSS) == 12 + 4
    assert lib.ekv_score_size(ctypes.byref(kv), 3) == 0
    bad = _kv(head_dim=96)
    assert lib.ekv_workspace_size(B.EKV_OP_ENTMAX_DECODE, ctypes.byref(bad), 0) == 0


def _topk(lib, kv, k=16, ub=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.ekv_select_topk(ctypes.byref(kv), ub, k, FAKE, FAKE, ws,
                               ws_bytes, None)


def test_validation_errors(lib):
    assert _topk(lib, _kv(), k=0) == B.EKV_ERR_INVALID_ARG
    assert _topk(lib, _kv(), ub=None) == B.EKV_ERR_INVALID_ARG
    assert _topk(lib, _kv(batch=0)) == B.EKV_ERR_INVALID_ARG
    assert _topk(lib, _kv(head_dim=96)) == B.EKV_ERR_UNSUPPORTED
    assert _topk(lib, _kv(page_size=8)) == B.EKV_ERR_UNSUPPORTED
    assert _topk(lib, _kv(group=3)) == B.EKV_ERR_UNSUPPORTED
    # one unit's float32 scores past 2 GiB - 64 KiB
    assert _topk(lib, _kv(group=8, page_size=64, max_pages=1 << 20)) == B.EKV_ERR_UNSUPPORTED
    assert _topk(lib, _kv(kv_dtype=7)) == B.EKV_ERR_INVALID_ARG
    assert _topk(lib, _kv(page_table=None)) == B.EKV_ERR_INVALID_ARG
    assert _topk(lib, _kv(), ws=None) == B.EKV_ERR_WORKSPACE
    assert _topk(lib, _kv(), ws_bytes=16) == B.EKV_ERR_WORKSPACE
    assert _topk(lib, _kv(), ws=FAKE + 64) == B.EKV_ERR_WORKSPACE
    assert "k must be >= 1" in (_topk(lib, _kv(), k=0) and
                                lib.ekv_last_error().decode())
    kv = _kv()
    # alpha must exceed 1; the Gaussian selector is built for 1.1 <= alpha <= 2
    for alpha, want in [(1.0, B.EKV_ERR_INVALID_ARG), (0.5, B.EKV_ERR_INVALID_ARG),
                        (float("nan"), B.EKV_ERR_INVALID_ARG),
                        (1.05, B.EKV_ERR_UNSUPPORTED), (2.5, B.EKV_ERR_UNSUPPORTED)]:
        assert lib.ekv_select_gauss(ctypes.byref(kv), FAKE, alpha, 0.5, FAKE,
                                    FAKE, FAKE, None, 0, None) == want
    assert lib.ekv_select_gauss(ctypes.byref(kv), FAKE, 1.5, -1.0, FAKE, FAKE,
                                FAKE, None, 0, None) == B.EKV_ERR_INVALID_ARG
    # decode: misaligned K, sel without count, non-positive scale, no output
    ws = 1 << 34
    assert lib.ekv_entmax_decode(ctypes.byref(_kv(k=FAKE + 2)), FAKE, 0.1, 1.5,
                                 None, None, None, FAKE, None, None, FAKE, ws,
                                 None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_entmax_decode(ctypes.byref(kv), FAKE, 0.1, 1.5, FAKE, None,
                                 None, FAKE, None, None, FAKE, ws,
                                 None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_entmax_decode(ctypes.byref(kv), FAKE, 0.0, 1.5, None, None,
                                 FAKE, FAKE, None, None, FAKE, ws,
                                 None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_entmax_decode(ctypes.byref(kv), FAKE, 0.1, 1.5, None, None,
                                 None, None, None, None, FAKE, ws,
                                 None) == B.EKV_ERR_INVALID_ARG
    # the decode without a workspace refuses a cache beyond its static scratch
    big = _kv(page_size=64, max_pages=16384)  # 1M tokens: 128 MiB of scores
    assert lib.ekv_entmax_decode_noalloc(ctypes.byref(big), FAKE, 0.1, 1.5, None,
                                         None, None, FAKE, None, None,
                                         None) == B.EKV_ERR_WORKSPACE
    # the single-launch decode: max_count >= 1, at most 2048 tokens on chip,
    # bfloat16 keys
    def small(kv_, max_count, out=FAKE):
        return lib.ekv_entmax_decode_small(ctypes.byref(kv_), FAKE, 0.1, 1.5,
                                           FAKE, FAKE, max_count, out, None,
                                           FAKE, 1 << 30, None)
    assert small(kv, 0) == B.EKV_ERR_INVALID_ARG
    assert small(kv, 65) == B.EKV_ERR_UNSUPPORTED  # 65 pages of 32 tokens
    assert small(_kv(kv_dtype=B.EKV_F32), 16) == B.EKV_ERR_UNSUPPORTED
    assert small(kv, 16, out=None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_entmax_decode_small(ctypes.byref(kv), FAKE, 0.1, 1.0, FAKE,
                                       FAKE, 16, FAKE, None, FAKE, 1 << 30,
                                       None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_entmax_decode_small(ctypes.byref(kv), FAKE, 0.1, 1.5, FAKE,
                                       FAKE, 16, FAKE, None, FAKE, 16,
                                       None) == B.EKV_ERR_WORKSPACE
    assert lib.ekv_softmax_decode(ctypes.byref(kv), FAKE, 0.1, None, None,
                                  FAKE, None, FAKE, 16,
                                  None) == B.EKV_ERR_WORKSPACE
    m = B.ekv_meta(None, None)
    assert lib.ekv_build_meta(ctypes.byref(kv), None, 0, ctypes.byref(m),
                              None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_score_pages(ctypes.byref(kv), ctypes.byref(B.ekv_meta(FAKE, None)),
                               FAKE, 0.1, B.EKV_SCORE_GAUSS, FAKE, None,
                               None) == B.EKV_ERR_INVALID_ARG
    assert lib.ekv_score_pages(ctypes.byref(kv), ctypes.byref(B.ekv_meta(FAKE, FAKE)),
                               FAKE, 0.1, 4, FAKE, FAKE,
                               None) == B.EKV_ERR_INVALID_ARG


def test_binding_refuses_missing_library(tmp_path):
    import importlib
    saved = B._lib_handle
    try:
        B._lib_handle = None
        with pytest.raises(RuntimeError, match="not built"):
            B.load_library(str(tmp_path / "missing.so"))
    finally:
        B._lib_handle = saved


@pytest.mark.parametrize("beta", [1.0, 4.0 / 3.0, 3.0, 9.0])
def test_gauss_jacobi_rule_is_exact_to_degree_2n_minus_1(beta):
    # int_{-1}^{1} (1 + x)^beta (1 + x)^j dx = 2^(beta+j+1) / (beta + j + 1):
    # every power of (1 + x) up to 2n - 1 is integrated exactly, i.e. every
    # polynomial of that degree
    n = 24
    x, w = B.ekv_quadrature_rule(B.EKV_RULE_JACOBI, beta, n)
    x, w = np.array(x), np.array(w)
    assert np.all(np.diff(x) > 0) and x[0] > -1 and x[-1] < 1 and np.all(w > 0)
    for j in range(2 * n):
        exact = 2.0 ** (beta + j + 1) / (beta + j + 1)
        got = float(np.sum(w * (1 + x) ** j))
        assert abs(got - exact) <= 1e-12 * exact, (j, got, exact)


def test_gauss_hermite_rule_moments():
    # E[X^k] of the standard normal: 0 for odd k, (k-1)!! for even k
    n = 16
    x, w = B.ekv_quadrature_rule(B.EKV_RULE_HERMITE, 0.0, n)
    x, w = np.array(x), np.array(w)
    assert np.allclose(x, -x[::-1], atol=1e-13) and abs(w.sum() - 1) < 1e-14
    df = 1.0
    for k in range(2 * n):
        got = float(np.sum(w * x ** k))
        if k % 2:
            assert abs(got) < 1e-9 * df
        else:
            if k:
                df *= k - 1
            assert abs(got - df) <= 1e-11 * df, (k, got, df)


def test_quadrature_rule_rejects_bad_input():
    with pytest.raises(B.EkvError):
        B.ekv_quadrature_rule(B.EKV_RULE_JACOBI, -1.5, 8)
    with pytest.raises(B.EkvError):
        B.ekv_quadrature_rule(7, 1.0, 8)
    with pytest.raises(B.EkvError):
        B.ekv_quadrature_rule(B.EKV_RULE_HERMITE, 0.0, 65)
