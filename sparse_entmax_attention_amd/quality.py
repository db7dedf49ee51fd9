"""Matched-budget quality of a page selection: entmax against softmax.

The Technical Summary's central comparison (§3, §4): a page set that covers
the entmax support loses nothing, because entmax gives zero weight to the
other tokens, while softmax weights every token and so loses mass on any
proper subset.  For the kept page set of every (sequence, KV head) -- the
selection held in ``DecodeBuffers.sel``/``count`` -- this measures, per query
head and with the same pages for both attentions:

  delta_entmax   full-cache entmax mass on the tokens outside the kept pages
                 (it bounds the output error by 2 B delta, B bounding the
                 value norms);
  delta_softmax  the same for softmax, 1 - exp(lse(kept) - lse(all));
  recall         share of the full-cache entmax support inside the kept
                 pages;
  err_entmax,    relative L2 distance between the output on the kept pages
  err_softmax    and the full-cache output.

Every attention result comes from the library's entry points: sparse and
full-cache entmax (the full-cache probabilities from its debug output) and
sparse and full-cache softmax with their log-sum-exp.  Only the sums and
norms that turn them into these numbers are tensor operations here; this is
evaluation code, not part of the decode step.
"""
from __future__ import annotations

import torch

from .decoder import DecodeBuffers


def kept_page_mask(buf: DecodeBuffers) -> torch.Tensor:
    """[batch][H_kv][max_pages] bool: the pages of each unit's selection."""
    MP = buf.kv.max_pages
    sel = buf.sel.long()
    valid = torch.arange(MP, device=sel.device) < buf.count.long()[..., None]
    sel = torch.where(valid, sel, torch.zeros_like(sel))
    kept = torch.zeros(sel.shape, dtype=torch.int32, device=sel.device)
    kept.scatter_add_(2, sel, valid.to(torch.int32))
    return kept > 0


def matched_budget_quality(buf: DecodeBuffers, q: torch.Tensor,
                           alpha: float) -> dict:
    """The five measures above, each a float64 tensor [batch][H_q].

    ``buf`` must hold a selection (``sel``/``count``, e.g. after
    ``select_topk`` or ``select_gauss``) and a softmax workspace
    (``DecodeBuffers(..., softmax=True)``).  Overwrites ``buf.out``,
    ``buf.tau`` and ``buf.lse``.
    """
    if buf.ws_softmax is None:
        raise ValueError("matched_budget_quality needs DecodeBuffers(softmax=True)")
    kv = buf.kv
    Bt, Hq, G = kv.batch, kv.num_q_heads, kv.group
    MP, P = kv.max_pages, kv.page_size
    probs = torch.empty(Bt, Hq, MP * P, dtype=torch.float32, device=kv.device)

    buf.entmax(q, alpha, selected=True)
    o_es = buf.out.double()
    buf.entmax(q, alpha, selected=False, probs=probs)
    o_ef = buf.out.double()
    buf.softmax(q, selected=True)
    o_ss, l_s = buf.out.double(), buf.lse.double()
    buf.softmax(q, selected=False)
    o_sf, l_f = buf.out.double(), buf.lse.double()

    kept = kept_page_mask(buf).repeat_interleave(G, dim=1)  # [B][Hq][MP]
    # the debug output is defined on the positions [0, seq_len) only
    pos = torch.arange(MP * P, device=kv.device)
    live = pos[None, :] < kv.seq_lens.long()[:, None]  # [B][MP*P]
    p = torch.where(live[:, None, :], probs, torch.zeros_like(probs))
    p = p.view(Bt, Hq, MP, P).double()
    page_mass = p.sum(-1)
    page_support = (p > 0).sum(-1).double()
    total = page_mass.sum(-1)
    dropped = torch.where(kept, torch.zeros_like(page_mass), page_mass).sum(-1)
    n_supp = page_support.sum(-1)
    inside = torch.where(kept, page_support, torch.zeros_like(page_support)).sum(-1)

    def rel(a, b):
        return (a - b).norm(dim=-1) / b.norm(dim=-1)

    return {
        "delta_entmax": dropped / total,
        "delta_softmax": -torch.expm1(l_s - l_f),
        "recall": inside / n_supp.clamp(min=1.0),
        "err_entmax": rel(o_es, o_ef),
        "err_softmax": rel(o_ss, o_sf),
    }
