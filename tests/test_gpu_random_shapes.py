"""GPU parity over seeded random shapes: whole decode steps through the C ABI
against the fp64 oracle.

Each case draws, from its own seed, the batch, KV-head count, group size,
head_dim, page size, KV dtype, ragged lengths (drawn from one token up),
key distribution, alpha, selector and its parameter, so that the
kernels' index arithmetic meets combinations the named workloads do not.  In
some cases one token is appended after the metadata build and the step runs
with the tail refresh inside the scoring launch.  Every case checks the
selection, tau, the entmax output over the selection, softmax over the same
pages (with its log-sum-exp) and full-cache entmax.  Sizes stay small enough
for the oracle to finish each case in about a second.
"""
import random

import numpy as np
import pytest
import torch

import oracle as O
import sparse_entmax_attention_amd as ekv
import workloads
from parity_utils import (OUT_RTOL_L2, TAU_ATOL, HostCopy,
                          check_gauss_selection, check_topk_selection, f64,
                          paged_kv, rel_l2, scale_of)

pytestmark = pytest.mark.gpu

SEEDS = list(range(700, 724))


def draw(seed):
    r = random.Random(seed)
    spec = workloads.workload(
        "ragged_pool_b16",
        batch=r.randint(1, 4), num_kv_heads=r.choice([1, 2, 3]),
        group=r.choice([1, 2, 4, 8]), head_dim=r.choice([64, 128]),
        page_size=r.choice([16, 32, 64]), kv_dtype=r.choice(["f32", "bf16"]),
        len_range=(1, r.choice([200, 2000, 5000])),
        keys=r.choice(["clusters", "page_offset"]), needles=r.choice([0, 5]),
        n_clusters=r.choice([4, 16]), permute_slots=True, spare_pages=1)
    case = dict(alpha=r.choice([1.5, 2.0, 1.25]),
                selector=r.choice(["topk", "gauss"]),
                k=r.randint(1, 48), delta=r.choice([0.0, 0.5, 2.0]),
                append=r.random() < 0.5)
    return spec, case


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_step(gpu, seed):
    spec, c = draw(seed)
    alpha = c["alpha"]
    print("[case] random shape seed=%d spec=%s case=%s" % (seed, spec, c),
          flush=True)
    inp = workloads.generate(spec, seed, gpu)
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv, softmax=True)
    buf.build_meta()
    if c["append"]:
        gen = torch.Generator(device=gpu)
        gen.manual_seed(seed)
        workloads.append_token(inp, gen)
    mode = ekv.EKV_SCORE_GAUSS if c["selector"] == "gauss" else ekv.EKV_SCORE_BBOX
    if c["append"]:
        buf.refresh_score(inp.q, mode)
    else:
        buf.score(inp.q, mode)
    if c["selector"] == "gauss":
        buf.select_gauss(alpha, c["delta"])
    else:
        buf.select_topk(c["k"])
    buf.entmax(inp.q, alpha)
    torch.cuda.synchronize()
    sel, cnt = buf.sel.cpu().numpy(), buf.count.cpu().numpy()
    tau, out = f64(buf.tau), f64(buf.out)
    tau_hat = f64(buf.tau_hat)
    buf.softmax(inp.q, selected=True)
    torch.cuda.synchronize()
    s_out, s_lse = f64(buf.out), f64(buf.lse)
    buf.entmax(inp.q, alpha, selected=False)
    torch.cuda.synchronize()
    f_tau, f_out = f64(buf.tau), f64(buf.out)

    host = HostCopy(inp)
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            N = keys.shape[0]
            n_tok = O.page_token_counts(N, P)
            kmin, kmax, mean, var = O.unit_metadata(keys, P)
            got = sel[b, h, :cnt[b, h]]
            assert cnt[b, h] >= 1 and (np.diff(got) > 0).all(), (b, h)
            if c["selector"] == "gauss":
                mu, s2 = zip(*[O.gauss_moments(qs[j], mean, var, sc)
                               for j in range(G)])
                mu, s2 = np.stack(mu), np.stack(s2)
                th = np.array([O.solve_tau_hat(mu[j], s2[j], n_tok, alpha)
                               for j in range(G)])
                for j in range(G):
                    assert abs(tau_hat[b, h * G + j] - th[j]) <= TAU_ATOL, (b, h, j)
                check_gauss_selection(got, mu, s2, n_tok, th, alpha, c["delta"])
            else:
                want = O.decode_unit(qs, keys, vals, P, sc, alpha, "topk",
                                     k=c["k"])
                check_topk_selection(got, want, c["k"])
            ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=got)
            toks = ref["tokens"]
            for j in range(G):
                hq = h * G + j
                assert abs(tau[b, hq] - ref["tau"][j]) <= TAU_ATOL, (b, h, j)
                assert rel_l2(out[b, hq], ref["out"][j]) <= OUT_RTOL_L2, (b, h, j)
                o, lse = O.softmax_attend(qs[j], keys[toks], vals[toks], sc)
                assert rel_l2(s_out[b, hq], o) <= OUT_RTOL_L2, (b, h, j)
                assert abs(s_lse[b, hq] - lse) <= 1e-4 * max(1.0, abs(lse))
                z = (alpha - 1) * O.token_scores(qs[j], keys, sc)
                t = O.entmax_threshold(z, alpha)
                p = O.entmax_probs(z, t, alpha)
                assert abs(f_tau[b, hq] - t) <= TAU_ATOL, (b, h, j)
                assert rel_l2(f_out[b, hq], (p[:, None] * vals).sum(0)) <= OUT_RTOL_L2


# Many small units: more units than the key pass's staging area holds for
# its along-unit partition (G = 1, D = 64: 256), or more query heads than
# CUs (the selector's and threshold step's half-capacity forms), with
# sequences from one token up.
MANY = [
    dict(batch=300, num_kv_heads=1, group=1, head_dim=64, page_size=16, selector="gauss"),
    dict(batch=40, num_kv_heads=4, group=2, head_dim=128, page_size=32, selector="topk"),
]


@pytest.mark.parametrize("i", range(len(MANY)))
def test_many_small_units(gpu, i):
    m = dict(MANY[i])
    selector = m.pop("selector")
    alpha, delta, k = 1.5, 0.5, 6
    spec = workloads.workload("ragged_pool_b16", kv_dtype="bf16", len_range=(1, 300),
                              keys="clusters", needles=0, n_clusters=4,
                              permute_slots=True, spare_pages=1, **m)
    seed = 800 + i
    print("[case] many small units seed=%d spec=%s selector=%s" % (seed, spec, selector),
          flush=True)
    inp = workloads.generate(spec, seed, gpu)
    kv = paged_kv(inp)
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    if selector == "gauss":
        buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
        buf.select_gauss(alpha, delta)
    else:
        buf.score(inp.q, ekv.EKV_SCORE_BBOX)
        buf.select_topk(k)
    buf.entmax(inp.q, alpha)
    torch.cuda.synchronize()
    sel, cnt = buf.sel.cpu().numpy(), buf.count.cpu().numpy()
    tau, out, tau_hat = f64(buf.tau), f64(buf.out), f64(buf.tau_hat)
    buf.entmax(inp.q, alpha, selected=False)
    torch.cuda.synchronize()
    f_tau, f_out = f64(buf.tau), f64(buf.out)
    host = HostCopy(inp)
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            n_tok = O.page_token_counts(keys.shape[0], P)
            got = sel[b, h, :cnt[b, h]]
            assert cnt[b, h] >= 1 and (np.diff(got) > 0).all(), (b, h)
            if selector == "gauss":
                _, _, mean, var = O.unit_metadata(keys, P)
                mu, s2 = zip(*[O.gauss_moments(qs[j], mean, var, sc) for j in range(G)])
                mu, s2 = np.stack(mu), np.stack(s2)
                th = np.array([O.solve_tau_hat(mu[j], s2[j], n_tok, alpha) for j in range(G)])
                for j in range(G):
                    assert abs(tau_hat[b, h * G + j] - th[j]) <= TAU_ATOL, (b, h, j)
                check_gauss_selection(got, mu, s2, n_tok, th, alpha, delta)
            else:
                want = O.decode_unit(qs, keys, vals, P, sc, alpha, "topk", k=k)
                check_topk_selection(got, want, k)
            ref = O.decode_unit(qs, keys, vals, P, sc, alpha, "given", pages=got)
            for j in range(G):
                hq = h * G + j
                assert abs(tau[b, hq] - ref["tau"][j]) <= TAU_ATOL, (b, h, j)
                assert rel_l2(out[b, hq], ref["out"][j]) <= OUT_RTOL_L2, (b, h, j)
                z = (alpha - 1) * O.token_scores(qs[j], keys, sc)
                t = O.entmax_threshold(z, alpha)
                p = O.entmax_probs(z, t, alpha)
                assert abs(f_tau[b, hq] - t) <= TAU_ATOL, (b, h, j)
                assert rel_l2(f_out[b, hq], (p[:, None] * vals).sum(0)) <= OUT_RTOL_L2, (b, h, j)
