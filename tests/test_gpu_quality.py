"""GPU: softmax over a selection, and the matched-budget quality measures
(entmax against softmax on the same kept pages) against the oracle.

The selection is the GPU selector's own; the oracle evaluates the measures
on exactly those pages from fp64 copies of the device bytes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_entmax_attention_amd as ekv
import workloads
from parity_utils import OUT_RTOL_L2, HostCopy, f64, paged_kv, scale_of
from sparse_entmax_attention_amd.quality import matched_budget_quality

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides, seed, selector, alpha)
    "needle4k_topk": ("needle_4k_d64_f32", {}, 501, "topk", 1.5),
    "needle32k_topk_a2": ("needle_32k_gqa", {"seq_len": 32768 - 19}, 502, "topk", 2.0),
    "cluster_gauss": ("cluster_128k_b4", {"batch": 2, "seq_len": 9000}, 503, "gauss", 1.5),
}


def _run(name, gpu):
    wl, ov, seed, selector, alpha = CASES[name]
    spec = workloads.workload(wl, **ov)
    print("[case] %s seed %d" % (name, seed), flush=True)
    inp = workloads.generate(spec, seed, gpu)
    buf = ekv.DecodeBuffers(paged_kv(inp), softmax=True)
    buf.build_meta()
    if selector == "topk":
        buf.score(inp.q, ekv.EKV_SCORE_BBOX)
        buf.select_topk(spec.topk)
    else:
        buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
        buf.select_gauss(alpha, spec.delta)
    torch.cuda.synchronize()
    return spec, inp, buf, alpha


@pytest.mark.parametrize("name", list(CASES))
def test_selected_softmax(gpu, name):
    spec, inp, buf, _ = _run(name, gpu)
    buf.softmax(inp.q, selected=True)
    torch.cuda.synchronize()
    host = HostCopy(inp)
    out, lse = f64(buf.out), f64(buf.lse)
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            pages = buf.sel[b, h, :int(buf.count[b, h])].cpu().numpy()
            toks = O.pages_to_tokens(pages, keys.shape[0], P)
            for j in range(G):
                o, l = O.softmax_attend(qs[j], keys[toks], vals[toks], sc)
                d = out[b, h * G + j] - o
                assert np.linalg.norm(d) <= OUT_RTOL_L2 * np.linalg.norm(o)
                assert abs(lse[b, h * G + j] - l) <= 1e-4 * max(1.0, abs(l))


@pytest.mark.parametrize("name", list(CASES))
def test_matched_budget_quality(gpu, name):
    spec, inp, buf, alpha = _run(name, gpu)
    m = {k: v.cpu().numpy() for k, v in matched_budget_quality(buf, inp.q, alpha).items()}
    torch.cuda.synchronize()
    host = HostCopy(inp)
    P, G, sc = spec.page_size, spec.group, scale_of(spec)
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            qs, keys, vals = host.unit(b, h)
            pages = buf.sel[b, h, :int(buf.count[b, h])].cpu().numpy()
            ref = O.matched_budget_quality(qs, keys, vals, P, sc, alpha, pages)
            for j in range(G):
                hq = h * G + j
                _, p_full, _ = O.dropped_mass(qs[j], keys, [], sc, alpha)
                n_supp = int((p_full > 0).sum())
                assert abs(m["delta_entmax"][b, hq] - ref["delta_entmax"][j]) <= 1e-4
                assert abs(m["delta_softmax"][b, hq] - ref["delta_softmax"][j]) <= 1e-4
                # a token at the threshold may fall either side
                assert abs(m["recall"][b, hq] - ref["recall"][j]) <= 1.0 / n_supp + 1e-12
                assert abs(m["err_entmax"][b, hq] - ref["err_entmax"][j]) <= 1e-3
                assert abs(m["err_softmax"][b, hq] - ref["err_softmax"][j]) <= 1e-3
    # the comparison the pages draw: softmax always loses mass on a proper
    # subset, entmax only when the support is cut
    proper = (buf.count.cpu().numpy() <
              np.array([[(n + P - 1) // P] * spec.num_kv_heads for n in inp.lens]))
    proper_q = np.repeat(proper, G, axis=1)
    assert (m["delta_softmax"][proper_q] > 0).all()
    assert (m["delta_entmax"][m["recall"] == 1] <= 1e-6).all()
