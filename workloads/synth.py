"""Workload shapes and seeded generators for paged single-token decode.

Layout produced (the same one the library consumes):

* ``k``, ``v``: pool of physical page slots, ``[num_slots][H_kv][P][D]``, in
  the workload's KV dtype (float32 or bfloat16, rounded to nearest-even from
  float32 draws).
* ``page_table``: ``[B][max_pages]`` int32, logical page -> physical slot.
* ``seq_lens``: ``[B]`` int32, valid tokens per sequence.
* ``q``: ``[B][H_q][D]`` float32, query heads of KV head ``h`` are
  ``h*G .. h*G+G-1``.

Token slots that hold no valid token (the tail of a sequence's last page and
the spare pages kept for appends) are filled with large-magnitude noise so
that a kernel which reads past a sequence's end produces visibly wrong
results instead of plausible ones.

Two key distributions are drawn, following the workloads the EntmaxKV pages
evaluate on (needle retrieval and long-context clustered text):

* ``page_offset``: every key is N(0, I) plus one N(0, 0.5^2 I) offset vector
  shared by its page; queries are N(0, I); planted needle tokens have key
  3 q/|q| for the query head they are aligned with (round-robin over the G
  heads of the KV head).
* ``clusters``: per (sequence, KV head), 64 cluster means drawn N(0, I); the
  pages are cut into 64 contiguous runs (floor(n_pages/64) pages each, the
  remainder going to the last run) and every key of a run is its cluster mean
  plus N(0, 0.3^2 I) noise.  Each query head picks 1-3 distinct clusters
  uniformly and is the sum of their means divided by sqrt(count).  Needles,
  if any, are planted as above.

Values are N(0, I) in both.  The draws are taken in a fixed order from one
``torch.Generator`` seeded with ``seed`` on the target device, so one
(workload, seed, device) triple always yields the same bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
_GARBAGE_SCALE = 20.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one decode workload."""

    name: str
    batch: int
    num_kv_heads: int
    group: int
    head_dim: int
    page_size: int
    kv_dtype: str                      # "f32" or "bf16"
    seq_len: int = 0                   # fixed length of every sequence ...
    len_range: Optional[tuple] = None  # ... or ragged U{lo..hi} lengths
    keys: str = "page_offset"          # "page_offset" or "clusters"
    needles: int = 0                   # planted needle tokens per (b, KV head)
    n_clusters: int = 64
    permute_slots: bool = False        # physical slots randomly permuted
    spare_pages: int = 0               # free page-table entries per sequence
    alphas: tuple = (1.5,)
    selector: str = "topk"             # "topk", "gauss" or "all"
    topk: int = 0
    delta: float = 0.5

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.kv_dtype]


WORKLOADS = {
    # Single head, 4k tokens of fp32 K/V in pages of 16, bbox top-32, 8 needles.
    "needle_4k_d64_f32": Workload(
        name="needle_4k_d64_f32", batch=1, num_kv_heads=1, group=1, head_dim=64,
        page_size=16, kv_dtype="f32", seq_len=4096, keys="page_offset",
        needles=8, alphas=(1.5,), selector="topk", topk=32),
    # GQA 8x4, 32k bf16 tokens in pages of 32, bbox top-32 (1024-token budget),
    # 0.1 % of the tokens planted as needles (33 per KV head).
    "needle_32k_gqa": Workload(
        name="needle_32k_gqa", batch=1, num_kv_heads=8, group=4, head_dim=128,
        page_size=32, kv_dtype="bf16", seq_len=32768, keys="page_offset",
        needles=33, alphas=(1.5, 2.0), selector="topk", topk=32),
    # Batch 4 x 128k clustered tokens, pages of 32, Gaussian selector.
    "cluster_128k_b4": Workload(
        name="cluster_128k_b4", batch=4, num_kv_heads=8, group=4, head_dim=128,
        page_size=32, kv_dtype="bf16", seq_len=131072, keys="clusters",
        alphas=(1.5,), selector="gauss", delta=0.5),
    # 1M clustered tokens in pages of 64 with 100 needles per KV head: every
    # selector plus the full-cache softmax and entmax baselines.
    "cluster_1m": Workload(
        name="cluster_1m", batch=1, num_kv_heads=8, group=4, head_dim=128,
        page_size=64, kv_dtype="bf16", seq_len=1048576, keys="clusters",
        needles=100, alphas=(1.5,), selector="all", topk=16, delta=0.5),
    # 16 ragged sequences of U{16k..256k} tokens in one permuted pool of
    # 32-token pages; one token appended per sequence per step.
    "ragged_pool_b16": Workload(
        name="ragged_pool_b16", batch=16, num_kv_heads=8, group=4,
        head_dim=128, page_size=32, kv_dtype="bf16",
        len_range=(16384, 262144), keys="clusters", permute_slots=True,
        spare_pages=4, alphas=(1.5,), selector="gauss", delta=0.5),
}


def workload(name: str, **overrides) -> Workload:
    """Return the named workload, with any field replaced by ``overrides``."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


@dataclasses.dataclass
class PagedInputs:
    spec: Workload
    seed: int
    k: torch.Tensor            # [num_slots][H_kv][P][D]
    v: torch.Tensor            # [num_slots][H_kv][P][D]
    page_table: torch.Tensor   # [B][max_pages] int32
    seq_lens: torch.Tensor     # [B] int32
    q: torch.Tensor            # [B][H_q][D] float32
    lens: list                 # host copy of seq_lens
    cluster_means: Optional[torch.Tensor] = None  # [B][H_kv][C][D] float32
    needle_pos: Optional[list] = None              # [B][H_kv] -> LongTensor

    @property
    def num_slots(self) -> int:
        return self.k.shape[0]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


def _cluster_of_pages(n_pages: int, n_clusters: int, device) -> torch.Tensor:
    run = max(n_pages // n_clusters, 1)
    return torch.clamp(torch.arange(n_pages, device=device) // run,
                       max=n_clusters - 1)


def _draw_queries(spec: Workload, gen: torch.Generator, device,
                  means: Optional[torch.Tensor]) -> torch.Tensor:
    """Queries [B][H_q][D] for the workload's key distribution."""
    B, H, G, D = spec.batch, spec.num_kv_heads, spec.group, spec.head_dim
    if spec.keys == "page_offset":
        return torch.randn(B, H * G, D, generator=gen, device=device)
    q = torch.empty(B, H * G, D, device=device)
    for b in range(B):
        for h in range(H):
            for g in range(G):
                cnt = int(torch.randint(1, 4, (1,), generator=gen,
                                        device=device).item())
                pick = torch.randperm(spec.n_clusters, generator=gen,
                                      device=device)[:cnt]
                q[b, h * G + g] = means[b, h, pick].sum(0) / math.sqrt(cnt)
    return q


def generate(spec: Workload, seed: int, device="cpu") -> PagedInputs:
    """Draw the inputs of ``spec`` from ``seed`` on ``device``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, H, G, D, P = (spec.batch, spec.num_kv_heads, spec.group,
                     spec.head_dim, spec.page_size)

    if spec.len_range is not None:
        lo, hi = spec.len_range
        lens = torch.randint(lo, hi + 1, (B,), generator=gen,
                             device=device).tolist()
    else:
        lens = [spec.seq_len] * B
    n_pages = [(L + P - 1) // P for L in lens]
    own = [n + spec.spare_pages for n in n_pages]
    max_pages = max(own)
    num_slots = sum(own)
    if spec.permute_slots:
        slots = torch.randperm(num_slots, generator=gen, device=device)
    else:
        slots = torch.arange(num_slots, device=device)
    page_table = torch.zeros(B, max_pages, dtype=torch.int32, device=device)
    start = 0
    for b in range(B):
        page_table[b, :own[b]] = slots[start:start + own[b]].to(torch.int32)
        start += own[b]

    k = torch.randn(num_slots, H, P, D, generator=gen, device=device)
    k.mul_(_GARBAGE_SCALE)
    v = torch.randn(num_slots, H, P, D, generator=gen, device=device)
    v.mul_(_GARBAGE_SCALE)

    means = None
    if spec.keys == "clusters":
        means = torch.randn(B, H, spec.n_clusters, D, generator=gen,
                            device=device)
    q = _draw_queries(spec, gen, device, means)

    needle_pos = [[None] * H for _ in range(B)]
    for b in range(B):
        L, npg = lens[b], n_pages[b]
        pos = torch.arange(L, device=device)
        slot_of_tok = page_table[b, pos // P].long()
        off_of_tok = pos % P
        for h in range(H):
            if spec.keys == "page_offset":
                keys = torch.randn(L, D, generator=gen, device=device)
                offs = 0.5 * torch.randn(npg, D, generator=gen, device=device)
                keys += offs[pos // P]
            else:
                cl = _cluster_of_pages(npg, spec.n_clusters, device)
                keys = torch.randn(L, D, generator=gen, device=device)
                keys.mul_(0.3)
                keys += means[b, h][cl[pos // P]]
            vals = torch.randn(L, D, generator=gen, device=device)
            if spec.needles > 0:
                nn = min(spec.needles, L)
                npos = torch.randperm(L, generator=gen, device=device)[:nn]
                for j in range(nn):
                    qg = q[b, h * G + (j % G)]
                    keys[npos[j]] = 3.0 * qg / qg.norm()
                needle_pos[b][h] = npos.cpu()
            k[slot_of_tok, h, off_of_tok] = keys
            v[slot_of_tok, h, off_of_tok] = vals

    dt = spec.torch_dtype
    return PagedInputs(
        spec=spec, seed=seed, k=k.to(dt), v=v.to(dt), page_table=page_table,
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device), q=q,
        lens=list(lens), cluster_means=means, needle_pos=needle_pos)


def append_token(inp: PagedInputs, gen: torch.Generator) -> torch.Tensor:
    """Append one token to every sequence; returns first_page[B] (int32).

    The new key of each (sequence, KV head) is drawn from the sequence's last
    key cluster (clustered workloads) or N(0, I) (page-offset workloads); the
    value is N(0, I).  The row is written into the pool slot that the page
    table names for position ``seq_len``; ``seq_lens`` is advanced.  The
    returned array is the logical page holding the new token, i.e. the only
    page whose metadata changed.
    """
    spec = inp.spec
    B, H, D, P = spec.batch, spec.num_kv_heads, spec.head_dim, spec.page_size
    dev = inp.k.device
    first = []
    for b in range(B):
        pos = inp.lens[b]
        p = pos // P
        if p >= inp.max_pages:
            raise RuntimeError("sequence %d has no spare page for an append" % b)
        slot = int(inp.page_table[b, p].item())
        if spec.keys == "clusters":
            keys = inp.cluster_means[b, :, spec.n_clusters - 1] + 0.3 * torch.randn(
                H, D, generator=gen, device=dev)
        else:
            keys = torch.randn(H, D, generator=gen, device=dev)
        vals = torch.randn(H, D, generator=gen, device=dev)
        inp.k[slot, :, pos % P] = keys.to(inp.k.dtype)
        inp.v[slot, :, pos % P] = vals.to(inp.v.dtype)
        inp.lens[b] = pos + 1
        first.append(p)
    inp.seq_lens.copy_(torch.tensor(inp.lens, dtype=torch.int32))
    return torch.tensor(first, dtype=torch.int32, device=dev)


def draw_fresh_queries(inp: PagedInputs, gen: torch.Generator) -> None:
    """Replace ``inp.q`` in place by a fresh draw from the workload's rule."""
    inp.q.copy_(_draw_queries(inp.spec, gen, inp.q.device, inp.cluster_means))
