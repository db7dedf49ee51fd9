"""Device buffers for the EntmaxKV decode step, and the step itself.

:class:`DecodeBuffers` allocates (once) every output and workspace the entry
points need for one paged cache and calls them in pipeline order.  It holds
no arithmetic: each method is a sequence of C-ABI calls.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _binding as B

SMALL_TOKENS = 2048  # tokens per unit the single-launch decode holds on chip


class DecodeBuffers:
    """Outputs and workspaces of one paged cache's decode step.

    kv: a :class:`PagedKV`.  bbox / gauss select which metadata to keep.
    """

    def __init__(self, kv: B.PagedKV, bbox: bool = True, gauss: bool = True,
                 softmax: bool = False):
        self.kv = kv
        dev = kv.device
        S, H, D = kv.num_slots, kv.num_kv_heads, kv.head_dim
        Bt, Hq, MP = kv.batch, kv.num_q_heads, kv.max_pages
        self.scale = 1.0 / math.sqrt(D)
        self.bbox = torch.empty(S, H, 2, D, dtype=kv.k.dtype, device=dev) if bbox else None
        self.gauss = torch.empty(S, H, 2, D, dtype=torch.float32, device=dev) if gauss else None
        # ub / gstat hold the per-page values followed by 64-page tile
        # summaries; .ub and .gstat are views of the per-page part.
        self.ub_buf = self.ub = self.gstat_buf = self.gstat = None
        if bbox:
            self.ub_buf = torch.empty(B.ekv_score_size(kv, B.EKV_SCORE_BBOX),
                                      dtype=torch.float32, device=dev)
            self.ub = self.ub_buf[:Bt * Hq * MP].view(Bt, Hq, MP)
        if gauss:
            self.gstat_buf = torch.empty(B.ekv_score_size(kv, B.EKV_SCORE_GAUSS),
                                         dtype=torch.float32, device=dev)
            self.gstat = self.gstat_buf[:Bt * Hq * MP * 2].view(Bt, Hq, MP, 2)
        self.sel = torch.empty(Bt, H, MP, dtype=torch.int32, device=dev)
        self.count = torch.empty(Bt, H, dtype=torch.int32, device=dev)
        self.tau_hat = torch.empty(Bt, Hq, dtype=torch.float32, device=dev)
        self.tau = torch.empty(Bt, Hq, dtype=torch.float32, device=dev)
        self.out = torch.empty(Bt, Hq, D, dtype=torch.float32, device=dev)
        self.lse = torch.empty(Bt, Hq, dtype=torch.float32, device=dev)
        self.ws_topk = self._ws(B.EKV_OP_SELECT_TOPK)
        self.ws_gauss = self._ws(B.EKV_OP_SELECT_GAUSS)
        self.ws_decode = self._ws(B.EKV_OP_ENTMAX_DECODE)
        self.ws_softmax = self._ws(B.EKV_OP_SOFTMAX_DECODE) if softmax else None
        self.ws_small = None  # grown on demand, zero-filled (it holds counters)

    def _ws(self, op: int) -> Optional[torch.Tensor]:
        n = B.ekv_workspace_size(op, self.kv, 1)
        if n == 0:
            return None
        return torch.empty(n, dtype=torch.uint8, device=self.kv.device)

    # -- pipeline steps ------------------------------------------------------
    def build_meta(self, first_page=None, span_hint: int = 0, stream=None):
        B.ekv_build_meta(self.kv, self.bbox, self.gauss, first_page, span_hint,
                         stream)

    def score(self, q, mode: int, stream=None):
        B.ekv_score_pages(self.kv, self.bbox, self.gauss, q, self.scale, mode,
                          self.ub_buf if mode & B.EKV_SCORE_BBOX else None,
                          self.gstat_buf if mode & B.EKV_SCORE_GAUSS else None,
                          stream)

    def refresh_score(self, q, mode: int, stream=None):
        """The last page of every sequence gets fresh metadata, then every
        page is scored (one token appended per sequence since the last
        step)."""
        B.ekv_refresh_score_pages(self.kv, self.bbox, self.gauss, q, self.scale,
                                  mode,
                                  self.ub_buf if mode & B.EKV_SCORE_BBOX else None,
                                  self.gstat_buf if mode & B.EKV_SCORE_GAUSS else None,
                                  stream)

    def select_topk(self, k: int, stream=None):
        B.ekv_select_topk(self.kv, self.ub_buf, k, self.sel, self.count,
                          self.ws_topk, stream)

    def select_gauss(self, alpha: float, delta: float, stream=None):
        B.ekv_select_gauss(self.kv, self.gstat_buf, alpha, delta, self.sel,
                           self.count, self.tau_hat, self.ws_gauss, stream)

    def entmax(self, q, alpha: float, selected: bool = True, probs=None,
               stream=None, tau_hint=None):
        B.ekv_entmax_decode(self.kv, q, self.scale, alpha,
                            self.sel if selected else None,
                            self.count if selected else None, self.out,
                            self.tau, probs, self.ws_decode, stream,
                            tau_hint=tau_hint)

    def entmax_small(self, q, alpha: float, max_count: int, selected: bool = True,
                     stream=None):
        n = B.ekv_workspace_size(B.EKV_OP_ENTMAX_DECODE_SMALL, self.kv, max_count)
        if self.ws_small is None or self.ws_small.numel() < n:
            self.ws_small = torch.zeros(n, dtype=torch.uint8, device=self.kv.device)
        B.ekv_entmax_decode_small(self.kv, q, self.scale, alpha,
                                  self.sel if selected else None,
                                  self.count if selected else None, max_count,
                                  self.out, self.tau, self.ws_small, stream)

    def small_fits(self, max_count: int) -> bool:
        """Whether the single-launch decode takes selections of max_count pages."""
        return (self.kv.k.dtype == torch.bfloat16 and
                max_count * self.kv.page_size <= SMALL_TOKENS)

    def softmax(self, q, selected: bool = False, stream=None):
        B.ekv_softmax_decode(self.kv, q, self.scale,
                             self.sel if selected else None,
                             self.count if selected else None, self.out,
                             self.lse, self.ws_softmax, stream)

    # -- whole steps ---------------------------------------------------------
    def step_topk(self, q, alpha: float, k: int, stream=None, small=None):
        """Box scoring, top-k selection, then entmax over the kept pages: in
        one launch when the k pages fit on chip (``small``: None chooses,
        False forces the split decode)."""
        self.score(q, B.EKV_SCORE_BBOX, stream)
        self.select_topk(k, stream)
        n_keep = min(k, self.kv.max_pages)
        if small is None:
            small = self.small_fits(n_keep)
        if small:
            self.entmax_small(q, alpha, n_keep, True, stream)
        else:
            self.entmax(q, alpha, True, None, stream)

    def step_gauss(self, q, alpha: float, delta: float, stream=None,
                   hint: bool = True):
        """Gaussian selection, then entmax over the kept pages with the
        selector's threshold estimates as the decode's hint (``hint=False``
        decodes without it)."""
        self.score(q, B.EKV_SCORE_GAUSS, stream)
        self.select_gauss(alpha, delta, stream)
        self.entmax(q, alpha, True, None, stream,
                    tau_hint=self.tau_hat if hint else None)
