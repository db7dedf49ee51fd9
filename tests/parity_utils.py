"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and hand the oracle the exact bytes the GPU read."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import sparse_entmax_attention_amd as ekv

# Tolerances fixed by the task contract for this path (bf16 KV, fp32
# accumulation): tau and tau_hat within 1e-4 absolute, outputs within a
# relative L2 error of 2e-3, selections exact except pages whose ranking value
# lies within 1e-5 (relative, floor 1) of the cutoff.
TAU_ATOL = 1e-4
OUT_RTOL_L2 = 2e-3
CUT_REL = 1e-5


def paged_kv(inp) -> ekv.PagedKV:
    return ekv.PagedKV(inp.k, inp.v, inp.page_table, inp.seq_lens,
                       inp.spec.group)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a float32/bfloat16 device tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


class HostCopy:
    """The inputs as the oracle sees them (fp64 host arrays)."""

    def __init__(self, inp):
        self.spec = inp.spec
        self.k = f64(inp.k)
        self.v = f64(inp.v)
        self.pt = inp.page_table.cpu().numpy()
        self.lens = list(inp.lens)
        self.q = f64(inp.q)

    def unit(self, b, h):
        n = self.lens[b]
        keys = O.unit_tokens(self.k, self.pt[b], h, n)
        vals = O.unit_tokens(self.v, self.pt[b], h, n)
        G = self.spec.group
        return self.q[b, h * G:(h + 1) * G], keys, vals


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_topk_selection(gpu_sel, ref, k):
    """Selection equality up to pages within CUT_REL of the k-th value.

    ``ref`` is the oracle's ``decode_unit(..., "topk", k=k)`` result: its
    group values ``g`` (the largest box bound over the query heads) and its
    selection ``sel``."""
    ref_g = ref["g"]
    n = len(ref_g)
    want = set(int(x) for x in ref["sel"])
    got = set(int(x) for x in gpu_sel)
    assert len(got) == min(k, n)
    if got == want:
        return 0
    order = sorted(range(n), key=lambda p: (-ref_g[p], p))
    cut = ref_g[order[min(k, n) - 1]]
    tol = CUT_REL * max(abs(cut), 1.0)
    for p in got ^ want:
        assert abs(ref_g[p] - cut) <= tol, (p, ref_g[p], cut)
    return len(got ^ want)


def check_gauss_selection(gpu_sel, mu, s2, n_tok, tau_hat, alpha, delta):
    """Gaussian keep-set equality up to pages within CUT_REL of the cut.

    A page may differ between the two sets only when, for some head, its
    estimate lies within CUT_REL of that head's cut tau_hat - delta (the two
    sides may round it to opposite sides).  The one other allowed difference
    is the empty-selection fallback: a side that kept a single page not
    explained by a near cut must have kept the page with the largest margin
    max_h [(alpha-1) mhat_hp - tau_hat_h] (or one within CUT_REL of it).
    """
    ref = set(O.gauss_keep(mu, s2, n_tok, tau_hat, alpha, delta).tolist())
    got = set(int(x) for x in gpu_sel)
    if got == ref:
        return 0
    G = mu.shape[0]
    zhat = np.stack([(alpha - 1) * O.page_max_estimate(mu[h], s2[h], n_tok)
                     for h in range(G)])
    cuts = np.asarray(tau_hat, dtype=np.float64) - delta
    gap = np.max(zhat - np.asarray(tau_hat, dtype=np.float64)[:, None], axis=0)
    best = max(range(zhat.shape[1]), key=lambda p: (gap[p], -p))

    def near_cut(p):
        return any(abs(zhat[h, p] - cuts[h]) <= CUT_REL * max(abs(cuts[h]), 1.0)
                   for h in range(G))

    def fallback_page(p):
        return abs(gap[p] - gap[best]) <= CUT_REL * max(abs(gap[best]), 1.0)

    for p in got ^ ref:
        if near_cut(p):
            continue
        side = got if p in got else ref
        assert len(side) == 1 and fallback_page(p), (
            "page %d differs and is neither near a cut nor the fallback page "
            "(gpu %d pages, oracle %d)" % (p, len(got), len(ref)), zhat[:, p], tau_hat)
    return len(got ^ ref)


def scale_of(spec) -> float:
    return 1.0 / math.sqrt(spec.head_dim)
