"""ekv_entmax_decode_noalloc (static device scratch, no workspace argument)
against ekv_entmax_decode with a caller's workspace: the same kernels on the
same inputs, so tau and out must agree bit for bit (and hence within the
oracle tolerances).  Two calls in a row on one GPU, the second on a smaller
cache, so the second starts from the first one's leftovers in the scratch;
then a cache too large for the scratch is refused before any launch."""
import math

import pytest
import torch

import sparse_entmax_attention_amd as ekv
import workloads

pytestmark = pytest.mark.gpu


def _case(spec_name, overrides, seed, gpu):
    spec = workloads.workload(spec_name, **overrides)
    print("[case] no-alloc decode %s %s seed %d" % (spec_name, overrides, seed),
          flush=True)
    inp = workloads.generate(spec, seed, gpu)
    kv = ekv.PagedKV(inp.k, inp.v, inp.page_table, inp.seq_lens, spec.group)
    return spec, inp, kv


def _compare(spec, inp, kv, alpha, selector):
    buf = ekv.DecodeBuffers(kv)
    buf.build_meta()
    if selector == "topk":
        buf.score(inp.q, ekv.EKV_SCORE_BBOX)
        buf.select_topk(spec.topk or 16)
    else:
        buf.score(inp.q, ekv.EKV_SCORE_GAUSS)
        buf.select_gauss(alpha, spec.delta)
    buf.entmax(inp.q, alpha)
    want_out, want_tau = buf.out.clone(), buf.tau.clone()
    out = torch.full_like(buf.out, float("nan"))
    tau = torch.full_like(buf.tau, float("nan"))
    ekv.ekv_entmax_decode_noalloc(kv, inp.q, 1.0 / math.sqrt(spec.head_dim),
                                  alpha, buf.sel, buf.count, out, tau)
    torch.cuda.synchronize()
    assert torch.equal(tau, want_tau)
    assert torch.equal(out, want_out)
    # and the full cache, through the same scratch
    buf.entmax(inp.q, alpha, selected=False)
    want_out, want_tau = buf.out.clone(), buf.tau.clone()
    ekv.ekv_entmax_decode_noalloc(kv, inp.q, 1.0 / math.sqrt(spec.head_dim),
                                  alpha, None, None, out, tau)
    torch.cuda.synchronize()
    assert torch.equal(tau, want_tau)
    assert torch.equal(out, want_out)


def test_noalloc_decode_matches_workspace_decode(gpu):
    spec, inp, kv = _case("needle_32k_gqa", {}, 501, gpu)
    _compare(spec, inp, kv, 1.5, "topk")
    spec, inp, kv = _case("cluster_128k_b4", {"batch": 2, "seq_len": 9000}, 502, gpu)
    _compare(spec, inp, kv, 1.5, "gauss")


def test_noalloc_decode_refuses_a_cache_beyond_the_scratch(gpu):
    spec = workloads.workload("cluster_1m", seq_len=4096)
    inp = workloads.generate(spec, 503, gpu)
    # a page table as long as a 1M-token sequence: the decode workspace is
    # sized by max_pages and exceeds the static scratch
    big = torch.zeros(1, 16384, dtype=torch.int32, device=gpu)
    big[0, :inp.page_table.shape[1]] = inp.page_table[0]
    kv = ekv.PagedKV(inp.k, inp.v, big, inp.seq_lens, spec.group)
    assert ekv.ekv_workspace_size(ekv.EKV_OP_ENTMAX_DECODE, kv) > (64 << 20)
    out = torch.empty(1, spec.num_q_heads, spec.head_dim, device=gpu)
    with pytest.raises(ekv.EkvError) as e:
        ekv.ekv_entmax_decode_noalloc(kv, inp.q, 0.1, 1.5, None, None, out)
    assert e.value.status == 3  # EKV_ERR_WORKSPACE
