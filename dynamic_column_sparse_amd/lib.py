"""Thin ctypes binding of ``libchipmunk.so`` (argument marshalling only).

Each function has the C entry point's name and takes torch tensors (or None)
where the C call takes device pointers; every step of the computation runs in
the library's HIP kernels.  A missing library raises at import time: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .digest import source_digest

_HERE = os.path.dirname(os.path.abspath(__file__))
# CHIPMUNK_LIBRARY names another build of the same sources (the host-sanitized
# build of the test suite); it is held to the same ABI and source-digest check.
LIB_PATH = os.environ.get("CHIPMUNK_LIBRARY") or os.path.join(_HERE, "libchipmunk.so")

ABI_VERSION = 8
NOALLOC_SCRATCH_BYTES = 64 << 20   # CHIPMUNK_NOALLOC_SCRATCH_BYTES
ROW_BLOCK = 128
HEAD_DIM = 128
MLP, ATTN = 0, 1
ATTN_SPARSE, ATTN_REFRESH = 0, 1
MLP_RESCORE = 1   # chipmunk_mlp.flags: sparse steps rescore their recomputed units
MLP_FP8 = 2       # chipmunk_mlp.flags: the first product runs on fp8 operands
MLP_FP8_W2 = 4    # chipmunk_mlp.flags: the sparse delta's second product runs on fp8 operands
OP_DENSE_MLP, OP_SPARSE_MLP, OP_TOPK, OP_DENSE_ATTN, OP_SPARSE_ATTN = 0, 1, 2, 3, 4
OP_DENSE_MLP_FP8, OP_SPARSE_MLP_FP8 = 5, 6

STATUS = {0: "CHIPMUNK_OK", 1: "CHIPMUNK_E_NULLPTR", 2: "CHIPMUNK_E_SHAPE", 3: "CHIPMUNK_E_UNSUPPORTED",
          4: "CHIPMUNK_E_ALIGN", 5: "CHIPMUNK_E_WORKSPACE", 6: "CHIPMUNK_E_HIP", 7: "CHIPMUNK_E_INTERNAL"}

EXPORTS = ("chipmunk_dense_step", "chipmunk_identify_topk", "chipmunk_check_index_sets", "chipmunk_sparse_mlp_delta",
           "chipmunk_sparse_attn_delta", "chipmunk_sparse_attn_reident", "chipmunk_sparse_step",
           "chipmunk_sparse_step_reident", "chipmunk_sparse_mlp_delta_noalloc",
           "chipmunk_cache_writeback", "chipmunk_quantize_fp8",
           "chipmunk_quantize_fp8_cols",
           "chipmunk_workspace_bytes",
           "chipmunk_last_error", "chipmunk_abi_version", "chipmunk_source_digest", "chipmunk_timing_enable", "chipmunk_timing_read",
           "chipmunk_kernel_count", "chipmunk_kernel_name")


class ChipmunkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class MLPLayer(ctypes.Structure):
    """``chipmunk_mlp``: sizes and device pointers of one MLP layer."""
    _fields_ = [("n", ctypes.c_int64), ("d", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w1t", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("a_cache", ctypes.c_void_p), ("score", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("w1t_f8", ctypes.c_void_p), ("w1t_scale", ctypes.c_void_p),
                ("w2_f8", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


class AttnLayer(ctypes.Structure):
    """``chipmunk_attn``: sizes and device pointers of one attention layer's cache."""
    _fields_ = [("n", ctypes.c_int64), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("m", ctypes.c_void_p), ("num", ctypes.c_void_p),
                ("den", ctypes.c_void_p), ("score", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -m dynamic_column_sparse_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "chipmunk_dense_step": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, vp, vp, sz, vp]),
        "chipmunk_identify_topk": (ctypes.c_int, [vp, i64, i64, i32, vp, vp, sz, vp]),
        "chipmunk_check_index_sets": (ctypes.c_int, [vp, i64, i32, i64, vp, vp]),
        "chipmunk_sparse_mlp_delta": (ctypes.c_int, [vp, vp, vp, i32, vp, vp, vp, sz, vp]),
        "chipmunk_sparse_mlp_delta_noalloc": (ctypes.c_int, [vp, vp, vp, i32, vp, vp, vp]),
        "chipmunk_sparse_attn_delta": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, ctypes.c_int, vp, vp]),
        "chipmunk_sparse_attn_reident": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]),
        "chipmunk_sparse_step": (ctypes.c_int, [vp, vp, vp, i32, vp, vp, vp, sz,
                                                 vp, vp, vp, vp, vp, i32, vp, vp]),
        "chipmunk_sparse_step_reident": (ctypes.c_int, [vp, vp, vp, i32, vp, vp, vp, sz,
                                                         vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]),
        "chipmunk_cache_writeback": (ctypes.c_int, [vp, vp, vp, i32, vp]),
        "chipmunk_quantize_fp8": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
        "chipmunk_quantize_fp8_cols": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
        "chipmunk_workspace_bytes": (sz, [ctypes.c_int, i64, i32, i32, i32]),
        "chipmunk_last_error": (ctypes.c_char_p, []),
        "chipmunk_abi_version": (ctypes.c_int, []),
        "chipmunk_source_digest": (ctypes.c_char_p, []),
        "chipmunk_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "chipmunk_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_int64)]),
        "chipmunk_kernel_count": (ctypes.c_int, []),
        "chipmunk_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    # The library must be the build of the sources beside it: same ABI version,
    # same source digest.  A stale binary is refused, never run.
    ver = lib.chipmunk_abi_version()
    built = (lib.chipmunk_source_digest() or b"").decode()
    here = source_digest()
    if ver != ABI_VERSION or built != here:
        raise ImportError(f"{LIB_PATH} does not match the sources in this tree (ABI {ver}, sources {built}; "
                          f"expected ABI {ABI_VERSION}, sources {here}); rebuild it with "
                          "__graft_entry__.build() (python -m dynamic_column_sparse_amd.build)")
    return lib


_lib = _load()


def raw() -> ctypes.CDLL:
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def _check(rc: int):
    if rc != 0:
        raise ChipmunkError(rc, chipmunk_last_error())


def chipmunk_last_error() -> str:
    return (_lib.chipmunk_last_error() or b"").decode()


def chipmunk_abi_version() -> int:
    return _lib.chipmunk_abi_version()


def chipmunk_source_digest() -> str:
    return (_lib.chipmunk_source_digest() or b"").decode()


def chipmunk_workspace_bytes(op: int, n: int, d: int, h: int, k: int) -> int:
    return int(_lib.chipmunk_workspace_bytes(op, n, d, h, k))


def mlp_layer(n, d, h, w1t, w2, a_cache, score=None, b1=None, b2=None, flags=0, w1t_f8=None,
              w1t_scale=None, w2_f8=None, w2_scale=None) -> MLPLayer:
    return MLPLayer(n, d, h, _ptr(w1t), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(a_cache), _ptr(score), flags,
                    _ptr(w1t_f8), _ptr(w1t_scale), _ptr(w2_f8), _ptr(w2_scale))


def attn_layer(n, heads, m, num, den, score=None, scale=None, head_dim=HEAD_DIM) -> AttnLayer:
    if scale is None:
        scale = 1.0 / float(head_dim) ** 0.5
    return AttnLayer(n, heads, head_dim, scale, _ptr(m), _ptr(num), _ptr(den), _ptr(score))


def chipmunk_dense_step(kind: int, layer, x_or_q, k=None, v=None, out=None, ws=None, stream=None, ws_bytes=None):
    nbytes = _nbytes(ws, ws_bytes)
    _check(_lib.chipmunk_dense_step(kind, ctypes.byref(layer), _ptr(x_or_q), _ptr(k), _ptr(v), _ptr(out),
                                    _ptr(ws), nbytes, _stream(stream)))


def chipmunk_check_index_sets(idx, rows: int, k: int, cols: int, result, stream=None):
    """Enqueue the device check of index sets idx [rows][k] against the
    contract (values in [0, cols), rows strictly ascending); result is an int64
    device tensor of 2 that receives (rows breaking it, smallest such row or
    `rows`)."""
    _check(_lib.chipmunk_check_index_sets(_ptr(idx), rows, k, cols, _ptr(result), _stream(stream)))


def chipmunk_identify_topk(score, rows: int, cols: int, k: int, idx, ws=None, stream=None, ws_bytes=None):
    nbytes = _nbytes(ws, ws_bytes)
    _check(_lib.chipmunk_identify_topk(_ptr(score), rows, cols, k, _ptr(idx), _ptr(ws), nbytes, _stream(stream)))


def chipmunk_sparse_mlp_delta(layer: MLPLayer, x, idx, k: int, y, a_new_packed=None, ws=None, stream=None, ws_bytes=None):
    nbytes = _nbytes(ws, ws_bytes)
    _check(_lib.chipmunk_sparse_mlp_delta(ctypes.byref(layer), _ptr(x), _ptr(idx), k, _ptr(y), _ptr(a_new_packed),
                                          _ptr(ws), nbytes, _stream(stream)))


def chipmunk_sparse_mlp_delta_noalloc(layer: MLPLayer, x, idx, k: int, y, a_new_packed=None, stream=None):
    _check(_lib.chipmunk_sparse_mlp_delta_noalloc(ctypes.byref(layer), _ptr(x), _ptr(idx), k, _ptr(y),
                                                  _ptr(a_new_packed), _stream(stream)))


def chipmunk_sparse_attn_delta(layer: AttnLayer, q, k, v, idx, kk: int, mode: int, o=None, stream=None):
    _check(_lib.chipmunk_sparse_attn_delta(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), kk, mode,
                                           _ptr(o), _stream(stream)))


def chipmunk_sparse_attn_reident(layer: AttnLayer, q_prev, k_prev, v_prev, q, k, v, idx, kk: int, o, stream=None):
    _check(_lib.chipmunk_sparse_attn_reident(ctypes.byref(layer), _ptr(q_prev), _ptr(k_prev), _ptr(v_prev), _ptr(q),
                                             _ptr(k), _ptr(v), _ptr(idx), kk, _ptr(o), _stream(stream)))


def chipmunk_sparse_step(mlp: MLPLayer, x, mlp_idx, k: int, y, a_new_packed, ws, attn: AttnLayer, q, kx, v,
                         attn_idx, kk: int, o, stream=None, ws_bytes=None):
    nbytes = _nbytes(ws, ws_bytes)
    _check(_lib.chipmunk_sparse_step(ctypes.byref(mlp), _ptr(x), _ptr(mlp_idx), k, _ptr(y), _ptr(a_new_packed),
                                     _ptr(ws), nbytes, ctypes.byref(attn), _ptr(q), _ptr(kx), _ptr(v),
                                     _ptr(attn_idx), kk, _ptr(o), _stream(stream)))


def chipmunk_sparse_step_reident(mlp: MLPLayer, x, mlp_idx, k: int, y, a_new_packed, ws, attn: AttnLayer, q_prev,
                                 k_prev, v_prev, q, kx, v, attn_idx, kk: int, o, stream=None, ws_bytes=None):
    nbytes = _nbytes(ws, ws_bytes)
    _check(_lib.chipmunk_sparse_step_reident(ctypes.byref(mlp), _ptr(x), _ptr(mlp_idx), k, _ptr(y),
                                             _ptr(a_new_packed), _ptr(ws), nbytes, ctypes.byref(attn), _ptr(q_prev),
                                             _ptr(k_prev), _ptr(v_prev), _ptr(q), _ptr(kx), _ptr(v), _ptr(attn_idx),
                                             kk, _ptr(o), _stream(stream)))


def chipmunk_quantize_fp8(src, rows: int, cols: int, dst, scale, stream=None):
    _check(_lib.chipmunk_quantize_fp8(_ptr(src), rows, cols, _ptr(dst), _ptr(scale), _stream(stream)))


def chipmunk_quantize_fp8_cols(src, rows: int, cols: int, dst, scale, stream=None):
    _check(_lib.chipmunk_quantize_fp8_cols(_ptr(src), rows, cols, _ptr(dst), _ptr(scale), _stream(stream)))


def chipmunk_cache_writeback(layer: MLPLayer, a_new_packed, idx, k: int, stream=None):
    _check(_lib.chipmunk_cache_writeback(ctypes.byref(layer), _ptr(a_new_packed), _ptr(idx), k, _stream(stream)))


def chipmunk_timing_enable(on: bool):
    _check(_lib.chipmunk_timing_enable(1 if on else 0))


def chipmunk_timing_read(kid: int):
    """(total_ms, launches) of kernel `kid` since the last enable."""
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    _check(_lib.chipmunk_timing_read(kid, ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value


def kernel_names() -> list:
    return [_lib.chipmunk_kernel_name(i).decode() for i in range(_lib.chipmunk_kernel_count())]
