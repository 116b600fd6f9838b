"""Thin ctypes binding of libmoonep_streams.so (include/moonep_streams.h): the plain memory
streams the benchmark measures its ceilings with.  Argument marshalling only; not part of
the hot path.  Raises if the library is not built."""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoonep_streams.so")
SHAPE_WAVE_2K, SHAPE_BLOCK_4K = 0, 1
EXPORTS = ("moonep_stream_read", "moonep_stream_write", "moonep_stream_copy",
           "moonep_rows_fanout", "moonep_rows_gather", "moonep_rows_update")

_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.moonep_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
    L.moonep_stream_write.argtypes = [vp, i64, i32, i32, vp]
    L.moonep_stream_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    L.moonep_rows_fanout.argtypes = [vp, i64, i32, vp, vp, i64, i32, i32, vp]
    L.moonep_rows_gather.argtypes = [vp, i64, i32, vp, i64, vp, i32, i32, vp]
    L.moonep_rows_update.argtypes = [vp, i64, i32, vp, vp, vp, i64, i32, vp]
    for f in EXPORTS:
        getattr(L, f).restype = i32
    _lib = L
    return L


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with {rc}")


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _s(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def read(buf, sink, shape=SHAPE_BLOCK_4K, policy=1):
    _check(lib().moonep_stream_read(_p(buf), buf.numel() * buf.element_size(), shape, policy,
                                    _p(sink), _s(buf)), "stream_read")


def write(buf, shape=SHAPE_BLOCK_4K, policy=1):
    _check(lib().moonep_stream_write(_p(buf), buf.numel() * buf.element_size(), shape, policy,
                                     _s(buf)), "stream_write")


def copy(src, dst, shape=SHAPE_BLOCK_4K, policy=1):
    assert src.numel() * src.element_size() == dst.numel() * dst.element_size()
    _check(lib().moonep_stream_copy(_p(src), _p(dst), src.numel() * src.element_size(), shape,
                                    policy, _s(src)), "stream_copy")


def fanout(rows, K, src, dst, read_src=True):
    """dst[rows[i*K + k]] = src[i] (or a pattern when read_src is False); 2-D row tensors."""
    n = rows.numel() // K
    assert rows.dtype == torch.int32 and rows.is_contiguous()
    assert (not read_src) or (src.shape[0] >= n and
                              src.shape[1] * src.element_size() == dst.shape[1] * dst.element_size())
    _check(lib().moonep_rows_fanout(_p(rows), n, K, _p(src) if read_src else ctypes.c_void_p(0),
                                    _p(dst), dst.shape[0], dst.shape[1] * dst.element_size(),
                                    int(read_src), _s(dst)), "rows_fanout")


def gather(rows, K, src, dst, write_dst=True):
    """dst[i] = XOR_k src[rows[i*K + k]] (or nothing written when write_dst is False)."""
    n = rows.numel() // K
    assert rows.dtype == torch.int32 and rows.is_contiguous() and dst.shape[0] >= n
    assert src.shape[1] * src.element_size() == dst.shape[1] * dst.element_size()
    _check(lib().moonep_rows_gather(_p(rows), n, K, _p(src), src.shape[0], _p(dst),
                                    src.shape[1] * src.element_size(), int(write_dst), _s(src)),
           "rows_gather")


def update(rows, K, src, a, b):
    """b[rows[i*K + k]] = a[rows[i*K + k]] ^ src[i]; 2-D row tensors, a and b alike."""
    n = rows.numel() // K
    assert rows.dtype == torch.int32 and rows.is_contiguous() and src.shape[0] >= n
    rb = src.shape[1] * src.element_size()
    assert a.shape == b.shape and a.dtype == b.dtype and a.shape[1] * a.element_size() == rb
    _check(lib().moonep_rows_update(_p(rows), n, K, _p(src), _p(a), _p(b), a.shape[0], rb, _s(a)),
           "rows_update")
