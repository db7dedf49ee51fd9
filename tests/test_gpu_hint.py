"""The decode's threshold hint (tau_hint): whatever its value, the decode must
match the oracle on the same selection.  A hint from the Gaussian selector
takes the fast path (only scores above hint - 1/32 kept, checked by the
normalisation over them); a hint too high fails that check and the head is
recomputed; a hint far too low keeps more scores than fit on chip and is
recomputed too; NaN hints mark heads that take the plain path.  Results are
also compared with the unhinted decode of the same selection."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_entmax_attention_amd as ekv
import workloads
from parity_utils import (OUT_RTOL_L2, TAU_ATOL, HostCopy, f64, paged_kv,
                          rel_l2, scale_of)

pytestmark = pytest.mark.gpu

CASES = {
    "cluster_p32_ragged": ("cluster_128k_b4", {"batch": 2, "seq_len": 9000}, 701),
    "cluster_p64": ("cluster_1m", {"seq_len": 65536 + 3, "num_kv_heads": 3}, 702),
    "pool_permuted": ("ragged_pool_b16", {"batch": 3, "len_range": (700, 6000)}, 703),
    "gqa2_d64_p16": ("needle_32k_gqa", {"seq_len": 5000, "group": 2, "head_dim": 64,
                                         "page_size": 16, "num_kv_heads": 3,
                                         "needles": 9}, 704),
    "gqa8": ("cluster_128k_b4", {"batch": 1, "seq_len": 7000, "group": 8,
                                  "num_kv_heads": 2}, 705),
}
_cache = {}


def _inputs(name, gpu):
    if name not in _cache:
        wl, ov, seed = CASES[name]
        spec = workloads.workload(wl, **ov)
        print("[case] hint %s seed=%d %s" % (name, seed, ov), flush=True)
        inp = workloads.generate(spec, seed, gpu)
        _cache[name] = (inp, HostCopy(inp))
    return _cache[name]


def _hint(kind, tau_hat):
    h = tau_hat.clone()
    if kind == "high":
        h += 0.75
    elif kind == "low":
        h -= 50.0
    elif kind == "plus_inf":
        h.fill_(math.inf)
    elif kind == "nan_mixed":
        h.view(-1)[::2] = math.nan
    return h


def _check(buf, host, inp, alpha, tau, out, sel=None):
    spec = inp.spec
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    cnt = buf.count.cpu().numpy()
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            if sel is None:
                pages = np.arange((keys.shape[0] + P - 1) // P)
            else:
                pages = sel[b, h, :cnt[b, h]]
            ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=pages)
            for j in range(G):
                hq = h * G + j
                assert abs(tau[b, hq] - ref["tau"][j]) <= TAU_ATOL, (b, h, j)
                assert rel_l2(out[b, hq], ref["out"][j]) <= OUT_RTOL_L2, (b, h, j)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("kind", ["selector", "high", "low", "plus_inf", "nan_mixed"])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_hinted_selected_decode(gpu, name, kind, alpha):
    inp, host = _inputs(name, gpu)
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
    buf.select_gauss(alpha, inp.spec.delta)
    buf.entmax(inp.q, alpha)  # no hint
    torch.cuda.synchronize()
    plain_tau, plain_out = buf.tau.clone(), buf.out.clone()
    hint = _hint(kind, buf.tau_hat)
    buf.entmax(inp.q, alpha, tau_hint=hint)
    torch.cuda.synchronize()
    tau, out = f64(buf.tau), f64(buf.out)
    # the same selection decoded with and without the hint: equal up to the
    # order of the support sums, or, where a head was recomputed, up to the
    # float32 rounding of its scores (recomputed on the vector units, not the
    # matrix cores; sparsemax passes that rounding straight to the output)
    assert torch.allclose(buf.tau, plain_tau, rtol=0, atol=1e-5)
    assert (torch.linalg.vector_norm(buf.out - plain_out, dim=-1)
            <= 1e-4 * torch.linalg.vector_norm(plain_out, dim=-1)).all()
    _check(buf, host, inp, alpha, tau, out, buf.sel.cpu().numpy())
    # run to run, the hinted decode is bit for bit the same
    buf.entmax(inp.q, alpha, tau_hint=hint)
    torch.cuda.synchronize()
    assert torch.equal(torch.from_numpy(tau).float(), buf.tau.cpu())
    assert torch.equal(torch.from_numpy(out).float(), buf.out.cpu())


@pytest.mark.parametrize("name", ["cluster_p32_ragged", "pool_permuted", "gqa2_d64_p16"])
@pytest.mark.parametrize("kind", ["selector", "high", "low"])
def test_hinted_full_cache_decode(gpu, name, kind):
    # every page with the hint: a hinted key pass over the full cache, and
    # (low) heads whose kept scores do not fit on chip
    inp, host = _inputs(name, gpu)
    alpha = 1.5
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
    buf.select_gauss(alpha, inp.spec.delta)
    hint = _hint(kind, buf.tau_hat)
    buf.entmax(inp.q, alpha, selected=False, tau_hint=hint)
    torch.cuda.synchronize()
    _check(buf, host, inp, alpha, f64(buf.tau), f64(buf.out))


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_hint_with_candidates_beyond_lds(gpu, alpha):
    # Tiny keys put every score within a few thousandths: any hint below
    # them keeps all 12,779 tokens per head, more than fit on chip, so each
    # head is recomputed and solved as without a hint (and over the full
    # cache, finished by the apply step).
    D, P, npg, H, G = 128, 64, 200, 2, 4
    n = npg * P - 21
    print("[case] hint, candidates beyond LDS, alpha %g" % alpha, flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(77)
    k = (3e-4 * torch.randn(npg, H, P, D, generator=g)).to(torch.bfloat16).to(gpu)
    v = torch.randn(npg, H, P, D, generator=g).to(torch.bfloat16).to(gpu)
    pt = torch.randperm(npg, generator=g).to(torch.int32).reshape(1, npg).to(gpu)
    sl = torch.tensor([n], dtype=torch.int32, device=gpu)
    q = torch.randn(1, H * G, D, generator=g).to(gpu)
    kv = ekv.PagedKV(k, v, pt, sl, G)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    buf.score(q, ekv.EKV_SCORE_BBOX)
    buf.select_topk(npg)
    hint = torch.full((1, H * G), -1.0, device=gpu)
    buf.entmax(q, alpha, tau_hint=hint)
    torch.cuda.synchronize()
    sel_tau, sel_out = f64(buf.tau), f64(buf.out)
    buf.entmax(q, alpha, selected=False, tau_hint=hint)
    torch.cuda.synchronize()
    full_tau, full_out = f64(buf.tau), f64(buf.out)
    kh, vh, qh = f64(k), f64(v), f64(q)
    rows = pt.cpu().numpy()[0]
    sc = 1 / math.sqrt(D)
    for h in range(H):
        keys = kh[rows, h].reshape(-1, D)[:n]
        vals = vh[rows, h].reshape(-1, D)[:n]
        for j in range(G):
            hq = h * G + j
            z = (alpha - 1) * O.token_scores(qh[0, hq], keys, sc)
            assert (z > -1.0 - 1.0 / 32).all()
            t = O.entmax_threshold(z, alpha)
            p = O.entmax_probs(z, t, alpha)
            o = (p[:, None] * vals).sum(0)
            for tau_, out_ in ((sel_tau, sel_out), (full_tau, full_out)):
                assert abs(tau_[0, hq] - t) <= TAU_ATOL, (h, j)
                assert rel_l2(out_[0, hq], o) <= OUT_RTOL_L2, (h, j)


def test_hint_ignored_with_probabilities(gpu):
    # the debug probabilities need every score, so a hint is not used then
    inp, host = _inputs("pool_permuted", gpu)
    spec = inp.spec
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
    buf.select_gauss(1.5, spec.delta)
    probs = torch.full((spec.batch, spec.num_q_heads, inp.max_pages * spec.page_size),
                       -1.0, device=gpu)
    buf.entmax(inp.q, 1.5, probs=probs, tau_hint=buf.tau_hat + 0.75)
    torch.cuda.synchronize()
    pr = f64(probs)
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    sel, cnt = buf.sel.cpu().numpy(), buf.count.cpu().numpy()
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            pages = sel[b, h, :cnt[b, h]]
            toks = O.pages_to_tokens(pages, keys.shape[0], P)
            for j in range(G):
                z = (1.5 - 1) * O.token_scores(qs[j], keys[toks], sc)
                t = O.entmax_threshold(z, 1.5)
                p = O.entmax_probs(z, t, 1.5)
                got = pr[b, h * G + j, toks]
                assert np.abs(got - p).max() < 1e-4
