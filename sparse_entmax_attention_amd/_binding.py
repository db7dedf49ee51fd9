"""ctypes binding of libentmaxkv.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it turns torch tensors into device pointers, fills the
two host structs of the C ABI and raises :class:`EkvError` on a non-zero
status.  All compute runs in the HIP kernels of the library.  When the
library has not been built the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libentmaxkv.so")

EKV_OK = 0
EKV_ERR_INVALID_ARG = 1
EKV_ERR_UNSUPPORTED = 2
EKV_ERR_WORKSPACE = 3
EKV_ERR_HIP = 4

EKV_F32 = 0
EKV_BF16 = 1

EKV_SCORE_BBOX = 1
EKV_SCORE_GAUSS = 2

EKV_OP_SELECT_TOPK = 1
EKV_OP_SELECT_GAUSS = 2
EKV_OP_ENTMAX_DECODE = 3
EKV_OP_SOFTMAX_DECODE = 4
EKV_OP_ENTMAX_DECODE_SMALL = 5

_c_i32 = ctypes.c_int32
_c_f32 = ctypes.c_float
_c_p = ctypes.c_void_p
_c_size = ctypes.c_size_t


class ekv_paged_kv(ctypes.Structure):
    _fields_ = [
        ("batch", _c_i32), ("num_kv_heads", _c_i32), ("group", _c_i32),
        ("head_dim", _c_i32), ("page_size", _c_i32), ("num_slots", _c_i32),
        ("max_pages", _c_i32), ("kv_dtype", _c_i32),
        ("k", _c_p), ("v", _c_p), ("page_table", _c_p), ("seq_lens", _c_p),
    ]


class ekv_meta(ctypes.Structure):
    _fields_ = [("bbox", _c_p), ("gauss", _c_p)]


# name -> (restype, argtypes)
_SIGNATURES = {
    "ekv_build_meta": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_i32,
                                ctypes.POINTER(ekv_meta), _c_p]),
    "ekv_score_pages": (_c_i32, [ctypes.POINTER(ekv_paged_kv),
                                 ctypes.POINTER(ekv_meta), _c_p, _c_f32, _c_i32,
                                 _c_p, _c_p, _c_p]),
    "ekv_refresh_score_pages": (_c_i32, [ctypes.POINTER(ekv_paged_kv),
                                 ctypes.POINTER(ekv_meta), _c_p, _c_f32, _c_i32,
                                 _c_p, _c_p, _c_p]),
    "ekv_select_topk": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_i32,
                                 _c_p, _c_p, _c_p, _c_size, _c_p]),
    "ekv_select_gauss": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_f32,
                                  _c_f32, _c_p, _c_p, _c_p, _c_p, _c_size,
                                  _c_p]),
    "ekv_entmax_decode": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_f32,
                                   _c_f32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                   _c_p, _c_size, _c_p]),
    "ekv_entmax_decode_noalloc": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p,
                                           _c_f32, _c_f32, _c_p, _c_p, _c_p,
                                           _c_p, _c_p, _c_p, _c_p]),
    "ekv_entmax_decode_small": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p,
                                         _c_f32, _c_f32, _c_p, _c_p, _c_i32,
                                         _c_p, _c_p, _c_p, _c_size, _c_p]),
    "ekv_entmax_scores": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_f32,
                                   _c_f32, _c_p, _c_p, _c_p, _c_p, _c_size,
                                   _c_p]),
    "ekv_entmax_threshold": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_f32,
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_size,
                                      _c_p]),
    "ekv_entmax_apply": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_f32, _c_p,
                                  _c_p, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "ekv_softmax_decode": (_c_i32, [ctypes.POINTER(ekv_paged_kv), _c_p, _c_f32,
                                    _c_p, _c_p, _c_p, _c_p, _c_p, _c_size,
                                    _c_p]),
    "ekv_workspace_size": (_c_size, [_c_i32, ctypes.POINTER(ekv_paged_kv),
                                     _c_i32]),
    "ekv_read_probe": (_c_i32, [_c_p, _c_size, _c_p, _c_p]),
    "ekv_score_size": (_c_size, [ctypes.POINTER(ekv_paged_kv), _c_i32]),
    "ekv_quadrature_rule": (_c_i32, [_c_i32, ctypes.c_double, _c_i32,
                                     ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)]),
    "ekv_status_string": (ctypes.c_char_p, [_c_i32]),
    "ekv_last_error": (ctypes.c_char_p, []),
    "ekv_version": (_c_i32, []),
}

_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the library, with every signature declared."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(
            "libentmaxkv.so is not built (%s); run "
            "`python -m sparse_entmax_attention_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib_handle = lib
    return lib


class EkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(message)


def _check(status: int, name: str) -> None:
    if status != EKV_OK:
        lib = load_library()
        raise EkvError(status, "%s: %s (%s)" % (
            name, lib.ekv_status_string(status).decode(),
            lib.ekv_last_error().decode()))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DTYPE_CODES = {torch.float32: EKV_F32, torch.bfloat16: EKV_BF16}


class PagedKV:
    """A paged KV cache held in torch tensors.

    k, v: [num_slots][H_kv][P][D] (float32 or bfloat16); page_table:
    [B][max_pages] int32; seq_lens: [B] int32; group: query heads per KV head.
    """

    def __init__(self, k: torch.Tensor, v: Optional[torch.Tensor],
                 page_table: torch.Tensor, seq_lens: torch.Tensor, group: int):
        if k.dim() != 4:
            raise ValueError("k must be [num_slots][H_kv][P][D]")
        if k.dtype not in _DTYPE_CODES:
            raise ValueError("k must be float32 or bfloat16")
        if v is not None and (v.shape != k.shape or v.dtype != k.dtype):
            raise ValueError("v must match k in shape and dtype")
        if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
            raise ValueError("page_table and seq_lens must be int32")
        self.k, self.v = k, v
        self.page_table, self.seq_lens = page_table, seq_lens
        self.num_slots, self.num_kv_heads, self.page_size, self.head_dim = k.shape
        self.batch, self.max_pages = page_table.shape
        self.group = int(group)
        self.dtype_code = _DTYPE_CODES[k.dtype]

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def device(self):
        return self.k.device

    def struct(self) -> ekv_paged_kv:
        return ekv_paged_kv(
            self.batch, self.num_kv_heads, self.group, self.head_dim,
            self.page_size, self.num_slots, self.max_pages, self.dtype_code,
            _ptr(self.k), _ptr(self.v), _ptr(self.page_table),
            _ptr(self.seq_lens))


def _meta(bbox, gauss) -> ekv_meta:
    return ekv_meta(_ptr(bbox), _ptr(gauss))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def ekv_workspace_size(op: int, kv: PagedKV, k: int = 0) -> int:
    s = kv.struct()
    return int(load_library().ekv_workspace_size(op, ctypes.byref(s), k))


def ekv_score_size(kv: PagedKV, mode: int) -> int:
    s = kv.struct()
    return int(load_library().ekv_score_size(ctypes.byref(s), mode))


def ekv_build_meta(kv: PagedKV, bbox, gauss, first_page=None, span_hint=0,
                   stream=None) -> None:
    s, m = kv.struct(), _meta(bbox, gauss)
    _check(load_library().ekv_build_meta(ctypes.byref(s), _ptr(first_page),
                                         int(span_hint), ctypes.byref(m),
                                         _stream(stream)), "ekv_build_meta")


def ekv_score_pages(kv: PagedKV, bbox, gauss, q, scale: float, mode: int,
                    ub=None, gstat=None, stream=None) -> None:
    s, m = kv.struct(), _meta(bbox, gauss)
    _check(load_library().ekv_score_pages(
        ctypes.byref(s), ctypes.byref(m), _ptr(q), float(scale), int(mode),
        _ptr(ub), _ptr(gstat), _stream(stream)), "ekv_score_pages")


def ekv_refresh_score_pages(kv: PagedKV, bbox, gauss, q, scale: float,
                            mode: int, ub=None, gstat=None,
                            stream=None) -> None:
    """Rebuild every sequence's last-page metadata, then score the pages."""
    s, m = kv.struct(), _meta(bbox, gauss)
    _check(load_library().ekv_refresh_score_pages(
        ctypes.byref(s), ctypes.byref(m), _ptr(q), float(scale), int(mode),
        _ptr(ub), _ptr(gstat), _stream(stream)), "ekv_refresh_score_pages")


def ekv_select_topk(kv: PagedKV, ub, k: int, sel, count, ws,
                    stream=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_select_topk(
        ctypes.byref(s), _ptr(ub), int(k), _ptr(sel), _ptr(count), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)),
        "ekv_select_topk")


def ekv_select_gauss(kv: PagedKV, gstat, alpha: float, delta: float, sel,
                     count, tau_hat, ws=None, stream=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_select_gauss(
        ctypes.byref(s), _ptr(gstat), float(alpha), float(delta), _ptr(sel),
        _ptr(count), _ptr(tau_hat), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)),
        "ekv_select_gauss")


def ekv_entmax_decode(kv: PagedKV, q, scale: float, alpha: float, sel, count,
                      out, tau=None, probs=None, ws=None, stream=None,
                      tau_hint=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_entmax_decode(
        ctypes.byref(s), _ptr(q), float(scale), float(alpha), _ptr(sel),
        _ptr(count), _ptr(tau_hint), _ptr(out), _ptr(tau), _ptr(probs),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "ekv_entmax_decode")


def ekv_entmax_decode_noalloc(kv: PagedKV, q, scale: float, alpha: float, sel,
                              count, out, tau=None, probs=None,
                              stream=None, tau_hint=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_entmax_decode_noalloc(
        ctypes.byref(s), _ptr(q), float(scale), float(alpha), _ptr(sel),
        _ptr(count), _ptr(tau_hint), _ptr(out), _ptr(tau), _ptr(probs),
        _stream(stream)),
        "ekv_entmax_decode_noalloc")


def ekv_entmax_decode_small(kv: PagedKV, q, scale: float, alpha: float, sel,
                            count, max_count: int, out, tau=None, ws=None,
                            stream=None) -> None:
    """ws: ekv_workspace_size(EKV_OP_ENTMAX_DECODE_SMALL, kv, max_count)
    bytes, zero-filled before its first use (each call leaves it so)."""
    s = kv.struct()
    _check(load_library().ekv_entmax_decode_small(
        ctypes.byref(s), _ptr(q), float(scale), float(alpha), _ptr(sel),
        _ptr(count), int(max_count), _ptr(out), _ptr(tau), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)),
        "ekv_entmax_decode_small")


def ekv_entmax_scores(kv: PagedKV, q, scale: float, alpha: float, sel, count,
                      ws, stream=None, tau_hint=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_entmax_scores(
        ctypes.byref(s), _ptr(q), float(scale), float(alpha), _ptr(sel),
        _ptr(count), _ptr(tau_hint), _ptr(ws), ws.numel(), _stream(stream)),
        "ekv_entmax_scores")


def ekv_entmax_threshold(kv: PagedKV, alpha: float, sel, count, tau, out, ws,
                         stream=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_entmax_threshold(
        ctypes.byref(s), float(alpha), _ptr(sel), _ptr(count), _ptr(tau),
        _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "ekv_entmax_threshold")


def ekv_entmax_apply(kv: PagedKV, alpha: float, sel, count, out, probs, ws,
                     stream=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_entmax_apply(
        ctypes.byref(s), float(alpha), _ptr(sel), _ptr(count), _ptr(out),
        _ptr(probs), _ptr(ws), ws.numel(), _stream(stream)),
        "ekv_entmax_apply")


def ekv_softmax_decode(kv: PagedKV, q, scale: float, sel, count, out,
                       lse=None, ws=None, stream=None) -> None:
    s = kv.struct()
    _check(load_library().ekv_softmax_decode(
        ctypes.byref(s), _ptr(q), float(scale), _ptr(sel), _ptr(count),
        _ptr(out), _ptr(lse), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(stream)), "ekv_softmax_decode")


EKV_READ_PROBE_SINK = 8192


def ekv_read_probe(buf, sink, stream=None) -> None:
    """Stream all of ``buf`` (bytes a multiple of 16) through the read probe."""
    _check(load_library().ekv_read_probe(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
        _stream(stream)), "ekv_read_probe")


EKV_RULE_JACOBI = 0
EKV_RULE_HERMITE = 1


def ekv_quadrature_rule(kind: int, param: float, n: int):
    """Host-only: the (nodes, weights) lists of a Gauss rule used by the
    Gaussian selector at general alpha (EKV_RULE_JACOBI: weight (1+x)^param
    on [-1, 1]; EKV_RULE_HERMITE: the standard normal density)."""
    x = (ctypes.c_double * n)()
    w = (ctypes.c_double * n)()
    _check(load_library().ekv_quadrature_rule(kind, float(param), n, x, w),
           "ekv_quadrature_rule")
    return list(x), list(w)


def ekv_version() -> int:
    return int(load_library().ekv_version())
