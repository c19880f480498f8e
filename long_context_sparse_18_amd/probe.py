"""Thin ctypes binding of libsgqa_probe.so, the machine-peak probes the benchmark quotes its
rooflines against (argument marshalling only; the probes run in the library's HIP kernels).
Each function has the name of the C entry point without the ``sgqa_`` prefix and takes torch
device tensors.  If the library is not built the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .sgqa import OK, SgqaError, _need_cuda, _ptr, _stream

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsgqa_probe.so")
_lib = None

EXPORTS = ("sgqa_probe_mfma_bf16", "sgqa_probe_read", "sgqa_probe_gather",
           "sgqa_probe_last_error")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libsgqa_probe.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    lib.sgqa_probe_mfma_bf16.restype = st
    lib.sgqa_probe_mfma_bf16.argtypes = [i32, i32, p, p]
    lib.sgqa_probe_read.restype = st
    lib.sgqa_probe_read.argtypes = [p, sz, p, i32, p]
    lib.sgqa_probe_gather.restype = st
    lib.sgqa_probe_gather.argtypes = [p, i64, i32, p, i64, p, i32, p]
    lib.sgqa_probe_last_error.restype = ctypes.c_char_p
    lib.sgqa_probe_last_error.argtypes = []
    _lib = lib
    return lib


def check(status: int):
    if status != OK:
        raise SgqaError(status, load().sgqa_probe_last_error().decode())


def probe_mfma_bf16(sink, iters: int, stream=None):
    """Dense bf16 MFMA probe: sink.numel() waves, each iters x 8 32x32x16 products
    (32768 flop each); every sink entry becomes 2048 * iters."""
    _need_cuda(sink)
    if sink.dtype != torch.float32 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor (one entry per wave)")
    check(load().sgqa_probe_mfma_bf16(sink.numel(), iters, _ptr(sink), _stream(stream, sink)))


def probe_read(buf, sink, stream=None):
    """Streaming-read probe over the bytes of buf: sink (uint32 as int32, one entry per
    workgroup) receives partial word sums that add up mod 2^32 to the buffer's word sum."""
    _need_cuda(buf, sink)
    if not buf.is_contiguous() or sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError("buf must be contiguous and sink a contiguous int32 tensor")
    nbytes = buf.numel() * buf.element_size()
    check(load().sgqa_probe_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(),
                                 _stream(stream, buf)))


def probe_gather(table, idx, sink, stream=None):
    """Random-row gather probe: table [rows, row_bytes] (contiguous, any dtype), idx int32 [n]
    with entries in [0, rows); sink (int32, one entry per workgroup) receives partial word sums
    that add up mod 2^32 to the word sum of the gathered rows."""
    _need_cuda(table, idx, sink)
    if not table.is_contiguous() or idx.dtype != torch.int32 or sink.dtype != torch.int32:
        raise ValueError("table must be contiguous, idx and sink int32")
    rows = table.shape[0]
    row_bytes = table[0].numel() * table.element_size()
    if idx.numel() and (int(idx.min()) < 0 or int(idx.max()) >= rows):
        raise ValueError("idx entries must lie in [0, table rows)")
    check(load().sgqa_probe_gather(_ptr(table), rows, row_bytes, _ptr(idx), idx.numel(),
                                   _ptr(sink), sink.numel(), _stream(stream, table)))
