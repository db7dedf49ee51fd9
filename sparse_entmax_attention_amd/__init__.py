"""EntmaxKV support-aware paged decode for AMD MI355X (gfx950).

The compute runs in the HIP library ``libentmaxkv.so`` (C ABI declared in
``include/entmaxkv.h``); this package only marshals torch tensors into its
entry points (:mod:`._binding`) and owns the device buffers of a decode step
(:mod:`.decoder`).
"""
from ._binding import (  # noqa: F401
    EKV_BF16, EKV_F32, EKV_OP_ENTMAX_DECODE, EKV_OP_SELECT_GAUSS,
    EKV_OP_SELECT_TOPK, EKV_OP_SOFTMAX_DECODE, EKV_SCORE_BBOX,
    EKV_RULE_HERMITE, EKV_RULE_JACOBI, EKV_SCORE_GAUSS, EkvError, LIB_PATH,
    PagedKV, ekv_build_meta, ekv_quadrature_rule,
    ekv_entmax_apply, ekv_entmax_decode, ekv_entmax_decode_noalloc,
    ekv_entmax_decode_small,
    ekv_entmax_scores,
    EKV_READ_PROBE_SINK, ekv_entmax_threshold, ekv_read_probe,
    ekv_refresh_score_pages, ekv_score_pages, ekv_select_gauss,
    ekv_select_topk, ekv_score_size, ekv_softmax_decode, ekv_version, ekv_workspace_size,
    load_library,
)
from .decoder import DecodeBuffers  # noqa: F401
