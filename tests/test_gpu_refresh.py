"""The fused metadata refresh and scoring of a decode step
(ekv_refresh_score_pages) against the two calls it replaces,
ekv_build_meta(last page) followed by ekv_score_pages, bit for bit: the
refreshed metadata, the per-page scores and the tile summaries.

One token is appended to every sequence first, as in a decode loop.  The
cases cover the one-kernel form (every (sequence, KV head) gets a wave of its
own), the two-launch form it falls back to when there are more units than
resident waves, each scoring mode, float32 and bfloat16 keys, head sizes 64
and 128, page sizes 16 to 64, a sequence left empty and sequences whose last
page holds a single token.
"""
import pytest
import torch

import sparse_entmax_attention_amd as ekv
import workloads
from parity_utils import paged_kv

pytestmark = pytest.mark.gpu

BOTH = ekv.EKV_SCORE_BBOX | ekv.EKV_SCORE_GAUSS


def _buffers(kv):
    buf = ekv.DecodeBuffers(kv)
    buf.bbox.zero_()
    buf.gauss.zero_()
    buf.build_meta()
    return buf


def _check(spec, seed, gpu, modes=(BOTH,), empty=()):
    print("[case] %s seed %d batch %d" % (spec.name, seed, spec.batch), flush=True)
    inp = workloads.generate(spec, seed, gpu)
    kv = paged_kv(inp)
    a, b = _buffers(kv), _buffers(kv)
    gen = torch.Generator(device=gpu)
    gen.manual_seed(seed)
    first = workloads.append_token(inp, gen)
    for e in empty:  # an empty sequence: nothing to refresh or score
        inp.lens[e] = 0
    inp.seq_lens.copy_(torch.tensor(inp.lens, dtype=torch.int32))
    workloads.draw_fresh_queries(inp, gen)
    a.build_meta(first, span_hint=1)
    for mode in modes:
        for buf in (a, b):
            buf.ub_buf.zero_()
            buf.gstat_buf.zero_()
        a.score(inp.q, mode)
        b.refresh_score(inp.q, mode)
        torch.cuda.synchronize()
        assert torch.equal(a.bbox, b.bbox), mode
        assert torch.equal(a.gauss, b.gauss), mode
        if mode & ekv.EKV_SCORE_BBOX:
            assert torch.equal(a.ub_buf, b.ub_buf), mode
        if mode & ekv.EKV_SCORE_GAUSS:
            assert torch.equal(a.gstat_buf, b.gstat_buf), mode
    # and the pages of the non-empty sequences equal a full rebuild of the
    # appended cache
    c = _buffers(kv)
    torch.cuda.synchronize()
    P = spec.page_size
    used = torch.cat([inp.page_table[s, :(n + P - 1) // P].long()
                      for s, n in enumerate(inp.lens) if n > 0])
    assert torch.equal(b.bbox[used], c.bbox[used])
    assert torch.equal(b.gauss[used], c.gauss[used])


def test_refresh_ragged_bf16_all_modes(gpu):
    spec = workloads.workload("ragged_pool_b16", len_range=(1, 3000),
                              spare_pages=1)
    _check(spec, 401, gpu, modes=(BOTH, ekv.EKV_SCORE_GAUSS, ekv.EKV_SCORE_BBOX),
           empty=(3,))


def test_refresh_one_token_last_pages(gpu):
    # lengths that are multiples of the page size: the appended token opens
    # a new page holding only itself
    spec = workloads.workload("cluster_128k_b4", seq_len=4 * 64 * 32, batch=3,
                              spare_pages=1)
    _check(spec, 402, gpu)


def test_refresh_f32_d64_p16(gpu):
    spec = workloads.workload("needle_4k_d64_f32", batch=5, len_range=(1, 700),
                              needles=0, keys="clusters", spare_pages=1)
    _check(spec, 403, gpu)


def test_refresh_p64_gqa8(gpu):
    spec = workloads.workload("cluster_1m", seq_len=0, len_range=(100, 9000),
                              batch=3, group=8, needles=0, spare_pages=1)
    _check(spec, 404, gpu, modes=(BOTH, ekv.EKV_SCORE_GAUSS))


def test_refresh_more_units_than_waves(gpu):
    # 512 x 8 = 4096 units: more than the waves the device holds for the
    # fused kernel, so the refresh runs as a separate launch first
    spec = workloads.workload("ragged_pool_b16", batch=512, len_range=(1, 70),
                              page_size=16, spare_pages=1)
    _check(spec, 405, gpu, empty=(0, 511))
