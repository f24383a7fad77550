"""Python binding of libdsa.so, the MI355X (gfx950) DeepSeek Sparse Attention hot path.

The functions mirror the C ABI of include/dsa.h one to one and do argument
marshalling only: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.  Importing works without
the built library (so host-only code can inspect it); any call then raises
`DSALibraryMissing` -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "DSAError", "DSALibraryMissing", "Cache", "F32", "BF16", "E4M3", "LIB_PATH", "lib",
    "dsa_index_scores", "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_mla_decode",
    "dsa_sparse_mla_decode_workspace_size", "dsa_sparse_mla_prefill", "dsa_masked_mla_prefill",
    "dsa_index_topk", "dsa_index_topk_workspace_size", "dsa_indexer_quality",
    "dsa_indexer_quality_workspace_size",
    "dsa_cache_append", "dsa_sparse_mla_decode_noalloc", "dsa_noalloc_scratch_bytes",
    "dsa_read_probe", "dsa_read_probe_sink_words",
    "dsa_status_string", "dsa_check_indices", "dsa_check_block_table", "exported_symbols",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

F32, BF16, E4M3 = 0, 1, 2
_STATUS = ["DSA_OK", "DSA_ERR_NULL", "DSA_ERR_SHAPE", "DSA_ERR_DTYPE", "DSA_ERR_WORKSPACE",
           "DSA_ERR_LAUNCH", "DSA_ERR_UNSUPPORTED", "DSA_ERR_RANGE"]


class DSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        name = _STATUS[status] if 0 <= status < len(_STATUS) else f"status {status}"
        super().__init__(f"{fn} failed: {name}")


class DSALibraryMissing(RuntimeError):
    pass


class _Cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("seq_stride", ctypes.c_int64)]


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "dsa_index_scores": (_i32, [_i32, _vp, _vp, _vp, ctypes.POINTER(_Cache), _vp, _vp, _i32, _i32,
                                _i32, _vp, _i64, _vp]),
    "dsa_topk_workspace_size": (_sz, [_i32, _i64, _i32]),
    "dsa_topk": (_i32, [_vp, _i64, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "dsa_sparse_mla_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "dsa_sparse_mla_decode": (_i32, [_i32, _vp, ctypes.POINTER(_Cache), _vp, _i32, _i32, _i32, _i32,
                                     _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "dsa_sparse_mla_prefill": (_i32, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                      _vp, _vp]),
    "dsa_index_topk_workspace_size": (_sz, [_i32, _i64, _i32]),
    "dsa_index_topk": (_i32, [_i32, _vp, _vp, _vp, ctypes.POINTER(_Cache), _vp, _vp, _i32, _i32, _i32,
                              _i32, _vp, _vp, _sz, _vp]),
    "dsa_indexer_quality_workspace_size": (_sz, [_i32, _i32, _i64]),
    "dsa_indexer_quality": (_i32, [_vp, ctypes.POINTER(_Cache), _vp, _i64, _vp, _vp, _vp, _i32, _i32,
                                   _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_masked_mla_prefill": (_i32, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                      _vp, _vp]),
    "dsa_cache_append": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, ctypes.POINTER(_Cache),
                                ctypes.POINTER(_Cache), _vp]),
    "dsa_noalloc_scratch_bytes": (_sz, []),
    "dsa_sparse_mla_decode_noalloc": (_i32, [_i32, _vp, ctypes.POINTER(_Cache), _vp, _i32, _i32, _i32,
                                             _i32, _i32, _f32, _vp, _vp, _vp]),
    "dsa_read_probe_sink_words": (_i32, []),
    "dsa_read_probe": (_i32, [_vp, _i64, _vp, _vp]),
    "dsa_status_string": (ctypes.c_char_p, [_i32]),
    "dsa_check_indices": (_i32, [_vp, _i32, _i32, _vp, _i32, ctypes.POINTER(ctypes.c_int64)]),
    "dsa_check_block_table": (_i32, [_vp, _i32, _i32, _vp, _i32, _i64, ctypes.POINTER(ctypes.c_int64)]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libdsa.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DSALibraryMissing(
                f"{LIB_PATH} is not built; run long_context_sparse_06_amd.build.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


# --------------------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("DSA tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("DSA tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, st: int):
    if st != 0:
        raise DSAError(fn, st)


class Cache:
    """A contiguous or paged per-token cache (see dsa_cache in include/dsa.h)."""

    def __init__(self, data, scale=None, block_table=None, page_size: int = 0,
                 seq_stride: int = 0):
        self.data, self.scale, self.block_table = data, scale, block_table
        self.page_size = int(page_size)
        self.max_pages = int(block_table.shape[1]) if block_table is not None else 0
        self.seq_stride = int(seq_stride)

    def _c(self) -> _Cache:
        return _Cache(_ptr(self.data), _ptr(self.scale), _ptr(self.block_table), self.page_size,
                      self.max_pages, self.seq_stride)


# --------------------------------------------------------------------------- the ABI
def dsa_read_probe_sink_words() -> int:
    return int(lib().dsa_read_probe_sink_words())


def dsa_read_probe(buf, sink, stream=None):
    """Measurement only: streams `buf` (a device tensor, its size a multiple of 1024 bytes) once
    and writes per-workgroup XOR words to `sink` (uint32 [dsa_read_probe_sink_words()])."""
    _check("dsa_read_probe", lib().dsa_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                  _stream(stream)))


def dsa_status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def dsa_index_scores(dt: int, q, q_scale, w, keys: Cache, row_seq, row_pos, R: int, H_I: int,
                     d_I: int, scores, ld: int, stream=None):
    c = keys._c()
    _check("dsa_index_scores", lib().dsa_index_scores(
        dt, _ptr(q), _ptr(q_scale), _ptr(w), ctypes.byref(c), _ptr(row_seq), _ptr(row_pos), R, H_I,
        d_I, _ptr(scores), ld, _stream(stream)))


def dsa_topk_workspace_size(R: int, ld: int, k: int) -> int:
    return int(lib().dsa_topk_workspace_size(R, ld, k))


def dsa_topk(scores, ld: int, n_valid, R: int, k: int, idx, ws=None, ws_bytes: int = 0, stream=None):
    if ws is not None and not ws_bytes:
        ws_bytes = ws.numel() * ws.element_size()
    _check("dsa_topk", lib().dsa_topk(_ptr(scores), ld, _ptr(n_valid), R, k, _ptr(idx), _ptr(ws),
                                      ws_bytes, _stream(stream)))


def dsa_sparse_mla_decode_workspace_size(B: int, H: int, Dv: int, k: int) -> int:
    return int(lib().dsa_sparse_mla_decode_workspace_size(B, H, Dv, k))


def dsa_sparse_mla_decode(dt: int, q, kv: Cache, idx, B: int, H: int, Dqk: int, Dv: int, k: int,
                          softmax_scale: float, out, lse=None, ws=None, ws_bytes: int = 0,
                          stream=None):
    if ws is not None and not ws_bytes:
        ws_bytes = ws.numel() * ws.element_size()
    c = kv._c()
    _check("dsa_sparse_mla_decode", lib().dsa_sparse_mla_decode(
        dt, _ptr(q), ctypes.byref(c), _ptr(idx), B, H, Dqk, Dv, k, softmax_scale, _ptr(out),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_noalloc_scratch_bytes() -> int:
    return int(lib().dsa_noalloc_scratch_bytes())


def dsa_sparse_mla_decode_noalloc(dt: int, q, kv: Cache, idx, B: int, H: int, Dqk: int, Dv: int,
                                  k: int, softmax_scale: float, out, lse=None, stream=None):
    """dsa_sparse_mla_decode with its split partials in the library's static per-GPU array
    (no workspace, no allocation; overlapping calls on one GPU race)."""
    c = kv._c()
    _check("dsa_sparse_mla_decode_noalloc", lib().dsa_sparse_mla_decode_noalloc(
        dt, _ptr(q), ctypes.byref(c), _ptr(idx), B, H, Dqk, Dv, k, softmax_scale, _ptr(out),
        _ptr(lse), _stream(stream)))


def dsa_sparse_mla_prefill(dt: int, q, kv, idx, T: int, H: int, Dqk: int, Dv: int, k: int,
                           softmax_scale: float, out, lse=None, stream=None):
    _check("dsa_sparse_mla_prefill", lib().dsa_sparse_mla_prefill(
        dt, _ptr(q), _ptr(kv), _ptr(idx), T, H, Dqk, Dv, k, softmax_scale, _ptr(out), _ptr(lse),
        _stream(stream)))


def dsa_cache_append(k_new, kv_new, row_seq, row_pos, R: int, d_I: int, Dqk: int, keys: Cache,
                     kv: Cache, stream=None):
    """Writes each row's new token into the key cache (e4m3 + fp32 scale) and the latent
    cache, at slot (row_seq[r], row_pos[r])."""
    ck, cv = keys._c(), kv._c()
    _check("dsa_cache_append", lib().dsa_cache_append(
        _ptr(k_new), _ptr(kv_new), _ptr(row_seq), _ptr(row_pos), R, d_I, Dqk, ctypes.byref(ck),
        ctypes.byref(cv), _stream(stream)))


def dsa_masked_mla_prefill(dt: int, q, kv, idx, T: int, H: int, Dqk: int, Dv: int, k: int,
                           softmax_scale: float, out, lse=None, stream=None):
    """dsa_sparse_mla_prefill's result in dense masked form (positions 0..t, kept set as mask)."""
    _check("dsa_masked_mla_prefill", lib().dsa_masked_mla_prefill(
        dt, _ptr(q), _ptr(kv), _ptr(idx), T, H, Dqk, Dv, k, softmax_scale, _ptr(out), _ptr(lse),
        _stream(stream)))


def dsa_index_topk_workspace_size(R: int, n_max: int, k: int) -> int:
    return int(lib().dsa_index_topk_workspace_size(R, n_max, k))


def dsa_index_topk(dt: int, q, q_scale, w, keys: Cache, row_seq, row_pos, R: int, H_I: int,
                   d_I: int, k: int, idx, ws, ws_bytes: int = 0, stream=None):
    """Index scores and top-k in one call (n_valid = row_pos + 1); scores live in `ws`."""
    if ws is not None and not ws_bytes:
        ws_bytes = ws.numel() * ws.element_size()
    c = keys._c()
    _check("dsa_index_topk", lib().dsa_index_topk(
        dt, _ptr(q), _ptr(q_scale), _ptr(w), ctypes.byref(c), _ptr(row_seq), _ptr(row_pos), R, H_I,
        d_I, k, _ptr(idx), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_indexer_quality_workspace_size(R: int, H: int, ld: int) -> int:
    return int(lib().dsa_indexer_quality_workspace_size(R, H, ld))


def dsa_indexer_quality(q, kv: Cache, scores, ld: int, idx, row_seq, row_pos, R: int, H: int,
                        Dqk: int, k: int, softmax_scale: float, kl, recall, ws, ws_bytes: int = 0,
                        stream=None, kl_rev=None):
    """Per row: KL(dense head-averaged attention || softmax(index scores)), the kept set's
    dense attention mass, and (kl_rev, optional) KL in the other order."""
    if ws is not None and not ws_bytes:
        ws_bytes = ws.numel() * ws.element_size()
    c = kv._c()
    _check("dsa_indexer_quality", lib().dsa_indexer_quality(
        _ptr(q), ctypes.byref(c), _ptr(scores), ld, _ptr(idx), _ptr(row_seq), _ptr(row_pos), R, H,
        Dqk, k, softmax_scale, _ptr(kl), _ptr(recall), _ptr(kl_rev), _ptr(ws), ws_bytes,
        _stream(stream)))


def _host_i32(a):
    """A C-contiguous int32 numpy copy of a tensor (device tensors are copied to the host)."""
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def dsa_check_indices(idx, n_valid, strict: bool = False) -> None:
    """Host-side range check of kept-index lists idx [R, k] against n_valid [R] (device tensors
    are copied to the host first).  Raises DSAError (DSA_ERR_RANGE, with `first_bad` the flat
    index of the first offending entry) if an entry is out of range -- or, with strict, breaks
    the ascending, repeat-free, -1-padded form dsa_topk writes."""
    a, n = _host_i32(idx), _host_i32(n_valid)
    if a.ndim != 2 or n.shape != (a.shape[0],):
        raise ValueError("idx must be [R, k] and n_valid [R]")
    bad = ctypes.c_int64(-1)
    st = lib().dsa_check_indices(a.ctypes.data, a.shape[0], a.shape[1], n.ctypes.data, int(bool(strict)),
                                 ctypes.byref(bad))
    if st != 0:
        e = DSAError("dsa_check_indices", st)
        e.first_bad = int(bad.value)
        raise e


def dsa_check_block_table(table, lengths, page_size: int, pool_pages: int) -> None:
    """Host-side check that every page the sequences use (lengths [B] tokens) maps into a pool
    of pool_pages pages in table [B, max_pages].  Raises DSAError (DSA_ERR_RANGE, with
    `first_bad`: the flat table index, or -1 - b for an out-of-range length) otherwise."""
    t, ln = _host_i32(table), _host_i32(lengths)
    if t.ndim != 2 or ln.shape != (t.shape[0],):
        raise ValueError("table must be [B, max_pages] and lengths [B]")
    bad = ctypes.c_int64(-1)
    st = lib().dsa_check_block_table(t.ctypes.data, t.shape[0], t.shape[1], ln.ctypes.data, int(page_size),
                                     int(pool_pages), ctypes.byref(bad))
    if st != 0:
        e = DSAError("dsa_check_block_table", st)
        e.first_bad = int(bad.value)
        raise e
