"""GPU parity at the workloads' full sizes, on sampled units.

Every workload is generated at its full shape and the decode step runs for
all (sequence, KV head) units on the GPU, in the launch configuration the
benchmark uses.  The fp64 oracle then recomputes a few sampled units one by
one from copies of just those units' bytes (a whole 1M-token pool would not
fit the host in fp64).
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_entmax_attention_amd as ekv
import workloads
from parity_utils import (OUT_RTOL_L2, TAU_ATOL, check_gauss_selection,
                          check_topk_selection, f64, paged_kv, rel_l2,
                          scale_of)

pytestmark = pytest.mark.gpu


def unit_copy(inp, b, h):
    """fp64 host copies (qs [G][D], keys [N][D], vals [N][D]) of one unit,
    gathered through its page table on the device first."""
    spec = inp.spec
    P, D, G = spec.page_size, spec.head_dim, spec.group
    n = inp.lens[b]
    rows = inp.page_table[b, :(n + P - 1) // P].long()
    keys = inp.k[rows, h].reshape(-1, D)[:n].double().cpu().numpy()
    vals = inp.v[rows, h].reshape(-1, D)[:n].double().cpu().numpy()
    qs = inp.q[b, h * G:(h + 1) * G].double().cpu().numpy()
    return qs, keys, vals


def check_gauss_unit(buf, inp, b, h, alpha, delta):
    spec = inp.spec
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    qs, keys, vals = unit_copy(inp, b, h)
    _, _, mean, var = O.unit_metadata(keys, P)
    n_tok = O.page_token_counts(keys.shape[0], P)
    mu, s2 = zip(*[O.gauss_moments(qs[j], mean, var, sc) for j in range(G)])
    mu, s2 = np.stack(mu), np.stack(s2)
    th = np.array([O.solve_tau_hat(mu[j], s2[j], n_tok, alpha) for j in range(G)])
    tau_hat, tau, out = f64(buf.tau_hat), f64(buf.tau), f64(buf.out)
    for j in range(G):
        assert abs(tau_hat[b, h * G + j] - th[j]) <= TAU_ATOL, (b, h, j)
    cnt = int(buf.count[b, h].item())
    got = buf.sel[b, h, :cnt].cpu().numpy()
    assert cnt >= 1 and (np.diff(got) > 0).all()
    check_gauss_selection(got, mu, s2, n_tok, th, alpha, delta)
    ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=got)
    for j in range(G):
        hq = h * G + j
        assert abs(tau[b, hq] - ref["tau"][j]) <= TAU_ATOL, (b, h, j)
        assert rel_l2(out[b, hq], ref["out"][j]) <= OUT_RTOL_L2, (b, h, j)


def test_needle_32k_gqa_topk_all_units(gpu):
    spec = workloads.workload("needle_32k_gqa")
    print("[case] needle_32k_gqa full, seed 201", flush=True)
    inp = workloads.generate(spec, 201, gpu)
    buf = ekv.DecodeBuffers(paged_kv(inp))
    buf.build_meta()
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    for alpha in (1.5, 2.0):
        buf.step_topk(inp.q, alpha, spec.topk)
        torch.cuda.synchronize()
        tau, out = f64(buf.tau), f64(buf.out)
        for b in range(spec.batch):
            for h in range(spec.num_kv_heads):
                qs, keys, vals = unit_copy(inp, b, h)
                want = O.decode_unit(qs, keys, vals, P, sc, alpha, "topk",
                                     k=spec.topk)
                got = buf.sel[b, h, :int(buf.count[b, h].item())].cpu().numpy()
                check_topk_selection(got, want, spec.topk)
                ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=got)
                for j in range(G):
                    hq = h * G + j
                    assert abs(tau[b, hq] - ref["tau"][j]) <= TAU_ATOL
                    assert rel_l2(out[b, hq], ref["out"][j]) <= OUT_RTOL_L2


def test_cluster_128k_b4_gauss_sampled(gpu):
    spec = workloads.workload("cluster_128k_b4")
    print("[case] cluster_128k_b4 full, seed 202", flush=True)
    inp = workloads.generate(spec, 202, gpu)
    buf = ekv.DecodeBuffers(paged_kv(inp))
    buf.build_meta()
    alpha = spec.alphas[0]
    buf.step_gauss(inp.q, alpha, spec.delta)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 3), (2, 5), (3, 7)]:
        print("[unit] b=%d h=%d" % (b, h), flush=True)
        check_gauss_unit(buf, inp, b, h, alpha, spec.delta)


def test_cluster_1m_all_legs_sampled(gpu):
    spec = workloads.workload("cluster_1m")
    print("[case] cluster_1m full, seed 3000 (the benchmark's input)", flush=True)
    inp = workloads.generate(spec, 3000, gpu)
    buf = ekv.DecodeBuffers(paged_kv(inp), softmax=True)
    buf.build_meta()
    alpha = spec.alphas[0]
    P, G, sc = spec.page_size, spec.group, scale_of(spec)

    # Gaussian selector
    buf.step_gauss(inp.q, alpha, spec.delta)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (0, 5)]:
        print("[unit] gauss h=%d" % h, flush=True)
        check_gauss_unit(buf, inp, b, h, alpha, spec.delta)

    # top-16
    buf.step_topk(inp.q, alpha, spec.topk)
    torch.cuda.synchronize()
    tau, out = f64(buf.tau), f64(buf.out)
    for b, h in [(0, 1), (0, 6)]:
        print("[unit] topk h=%d" % h, flush=True)
        qs, keys, vals = unit_copy(inp, b, h)
        want = O.decode_unit(qs, keys, vals, P, sc, alpha, "topk", k=spec.topk)
        got = buf.sel[b, h, :int(buf.count[b, h].item())].cpu().numpy()
        check_topk_selection(got, want, spec.topk)
        ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=got)
        for j in range(G):
            assert abs(tau[b, h * G + j] - ref["tau"][j]) <= TAU_ATOL
            assert rel_l2(out[b, h * G + j], ref["out"][j]) <= OUT_RTOL_L2

    # full-cache entmax and softmax
    buf.entmax(inp.q, alpha, selected=False)
    torch.cuda.synchronize()
    tau, out = f64(buf.tau), f64(buf.out)
    b, h = 0, 2
    qs, keys, vals = unit_copy(inp, b, h)
    for j in range(G):
        o, t, _ = O.entmax_attend(qs[j], keys, vals, sc, alpha)
        assert abs(tau[b, h * G + j] - t) <= TAU_ATOL
        assert rel_l2(out[b, h * G + j], o) <= OUT_RTOL_L2
    buf.softmax(inp.q)
    torch.cuda.synchronize()
    out, lse = f64(buf.out), f64(buf.lse)
    b, h = 0, 7
    qs, keys, vals = unit_copy(inp, b, h)
    for j in range(G):
        o, l = O.softmax_attend(qs[j], keys, vals, sc)
        assert rel_l2(out[b, h * G + j], o) <= OUT_RTOL_L2
        assert abs(lse[b, h * G + j] - l) <= 1e-4 * max(1.0, abs(l))


def test_cluster_1m_pages_of_16_full_cache_sampled(gpu):
    """1M tokens in pages of 16: 524,288 page-heads, so every wave of the
    full-cache key pass and of the streaming softmax walks some 170 pages,
    several 64-page chunks of one unit (the query parts reloaded and the
    page records written per chunk; the softmax segment carried across
    chunks)."""
    spec = workloads.workload("cluster_1m", page_size=16)
    print("[case] cluster_1m, pages of 16, seed 3001", flush=True)
    inp = workloads.generate(spec, 3001, gpu)
    buf = ekv.DecodeBuffers(paged_kv(inp), softmax=True)
    alpha = spec.alphas[0]
    G, sc = spec.group, scale_of(spec)
    buf.entmax(inp.q, alpha, selected=False)
    torch.cuda.synchronize()
    tau, out = f64(buf.tau), f64(buf.out)
    b, h = 0, 3
    print("[unit] full-cache entmax h=%d" % h, flush=True)
    qs, keys, vals = unit_copy(inp, b, h)
    for j in range(G):
        o, t, _ = O.entmax_attend(qs[j], keys, vals, sc, alpha)
        assert abs(tau[b, h * G + j] - t) <= TAU_ATOL, j
        assert rel_l2(out[b, h * G + j], o) <= OUT_RTOL_L2, j
    buf.softmax(inp.q)
    torch.cuda.synchronize()
    out, lse = f64(buf.out), f64(buf.lse)
    b, h = 0, 4
    print("[unit] full-cache softmax h=%d" % h, flush=True)
    qs, keys, vals = unit_copy(inp, b, h)
    for j in range(G):
        o, l = O.softmax_attend(qs[j], keys, vals, sc)
        assert rel_l2(out[b, h * G + j], o) <= OUT_RTOL_L2, j
        assert abs(lse[b, h * G + j] - l) <= 1e-4 * max(1.0, abs(l)), j


def test_ragged_pool_b16_appends_sampled(gpu):
    spec = workloads.workload("ragged_pool_b16")
    print("[case] ragged_pool_b16 full, seed 204, 3 appends", flush=True)
    inp = workloads.generate(spec, 204, gpu)
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    gen = torch.Generator(device=gpu)
    gen.manual_seed(204)
    alpha = spec.alphas[0]
    for step in range(3):
        first = workloads.append_token(inp, gen)
        workloads.draw_fresh_queries(inp, gen)
        buf.build_meta(first, span_hint=1)
        buf.step_gauss(inp.q, alpha, spec.delta)
    torch.cuda.synchronize()
    # the refreshed tail pages equal a full rebuild, bit for bit
    full = ekv.DecodeBuffers(paged_kv(inp))
    full.build_meta()
    torch.cuda.synchronize()
    P = spec.page_size
    for b in range(spec.batch):
        tail = inp.page_table[b, (inp.lens[b] - 1) // P].long()
        assert torch.equal(buf.bbox[tail], full.bbox[tail])
        assert torch.equal(buf.gauss[tail], full.gauss[tail])
    for b, h in [(0, 0), (7, 4), (15, 7)]:
        print("[unit] b=%d h=%d len=%d" % (b, h, inp.lens[b]), flush=True)
        check_gauss_unit(buf, inp, b, h, alpha, spec.delta)


def test_cluster_1m_appended_fused_refresh_phases(gpu):
    # The 1M-token cache with one token appended (it opens a new 64-token
    # page), stepped the way the benchmark's Gaussian leg does it: the tail
    # page's refresh inside the scoring launch, then the selector and the
    # three decode phases as separate calls.
    spec = workloads.workload("cluster_1m", spare_pages=1)
    print("[case] cluster_1m + 1 token, seed 3001, fused refresh + phases",
          flush=True)
    inp = workloads.generate(spec, 3001, gpu)
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    gen = torch.Generator(device=gpu)
    gen.manual_seed(3001)
    workloads.append_token(inp, gen)
    workloads.draw_fresh_queries(inp, gen)
    alpha = spec.alphas[0]
    buf.refresh_score(inp.q, ekv.EKV_SCORE_GAUSS)
    buf.select_gauss(alpha, spec.delta)
    ekv.ekv_entmax_scores(kv, inp.q, buf.scale, alpha, buf.sel, buf.count,
                          buf.ws_decode)
    ekv.ekv_entmax_threshold(kv, alpha, buf.sel, buf.count, buf.tau, buf.out,
                             buf.ws_decode)
    ekv.ekv_entmax_apply(kv, alpha, buf.sel, buf.count, buf.out, None,
                         buf.ws_decode)
    torch.cuda.synchronize()
    assert inp.lens[0] == spec.seq_len + 1
    # the new page (one token) equals a full rebuild of it
    full = ekv.DecodeBuffers(paged_kv(inp))
    full.build_meta()
    torch.cuda.synchronize()
    tail = inp.page_table[0, spec.seq_len // spec.page_size].long()
    assert torch.equal(buf.bbox[tail], full.bbox[tail])
    assert torch.equal(buf.gauss[tail], full.gauss[tail])
    del full
    for b, h in [(0, 3), (0, 7)]:
        print("[unit] b=%d h=%d" % (b, h), flush=True)
        check_gauss_unit(buf, inp, b, h, alpha, spec.delta)
