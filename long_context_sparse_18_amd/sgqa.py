"""Thin ctypes binding of libsgqa.so (argument marshalling only).

Each function has the name of the C entry point without the ``sgqa_`` prefix
and takes torch device tensors; every step of the layer runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is not built the first call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .configs import LayerShape

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsgqa.so")
_lib = None

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)
OP_INDEXER_TOPK = 1
OP_ATTN_DECODE = 2
OP_ATTN_PREFILL = 3
OP_ATTN_BACKWARD = 4

EXPORTS = ("sgqa_index_build", "sgqa_index_build_from_keys", "sgqa_indexer_topk", "sgqa_sparse_attn_prefill",
           "sgqa_sparse_attn_decode", "sgqa_sparse_attn_decode_noalloc", "sgqa_swa_prefill", "sgqa_quantize_fp8",
           "sgqa_indexer_topk_fp8", "sgqa_sparse_attn_decode_fp8", "sgqa_sparse_attn_backward",
           "sgqa_workspace_bytes",
           "sgqa_status_string", "sgqa_last_error")


class Dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("proxy_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk_blocks", ctypes.c_int32)]

    @classmethod
    def of(cls, s: LayerShape) -> "Dims":
        return cls(s.num_q_heads, s.num_kv_heads, s.head_dim, s.proxy_dim, s.block_size,
                   s.topk_blocks)


class SgqaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libsgqa.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(Dims)
    st = ctypes.c_int
    lib.sgqa_index_build.restype = st
    lib.sgqa_index_build.argtypes = [dp, p, i64, p, i64, p, i32, i64, i64, p]
    lib.sgqa_index_build_from_keys.restype = st
    lib.sgqa_index_build_from_keys.argtypes = [dp, p, i64, p, p, i64, p, i32, i64, i64, p]
    lib.sgqa_indexer_topk.restype = st
    lib.sgqa_indexer_topk.argtypes = [dp, p, i64, p, i64, p, i32, i32, p, p, p, sz, p]
    lib.sgqa_sparse_attn_prefill.restype = st
    lib.sgqa_sparse_attn_prefill.argtypes = [dp, p, p, p, p, p, i64, i32, i64, ctypes.c_float, p,
                                             p, p, sz, p]
    lib.sgqa_sparse_attn_decode.restype = st
    lib.sgqa_sparse_attn_decode.argtypes = [dp, p, p, p, i64, p, p, p, i32, ctypes.c_float, p, p,
                                            p, sz, p]
    lib.sgqa_sparse_attn_decode_noalloc.restype = st
    lib.sgqa_sparse_attn_decode_noalloc.argtypes = [dp, p, p, p, i64, p, p, p, i32,
                                                    ctypes.c_float, p, p, p]
    lib.sgqa_swa_prefill.restype = st
    lib.sgqa_swa_prefill.argtypes = [dp, p, p, p, p, i64, i32, i64, i64, ctypes.c_float, p, p, p]
    lib.sgqa_quantize_fp8.restype = st
    lib.sgqa_quantize_fp8.argtypes = [p, i64, i32, p, p, p]
    lib.sgqa_indexer_topk_fp8.restype = st
    lib.sgqa_indexer_topk_fp8.argtypes = [dp, p, i64, p, p, i64, p, i32, p, p, p, sz, p]
    lib.sgqa_sparse_attn_decode_fp8.restype = st
    lib.sgqa_sparse_attn_decode_fp8.argtypes = [dp, p, p, p, p, p, i64, p, p, p, i32,
                                                ctypes.c_float, p, p, p, sz, p]
    lib.sgqa_sparse_attn_backward.restype = st
    lib.sgqa_sparse_attn_backward.argtypes = [dp, p, p, p, p, p, i64, i32, i64, ctypes.c_float, p,
                                              p, p, p, p, p, p, p, sz, i64, p]
    lib.sgqa_workspace_bytes.restype = sz
    lib.sgqa_workspace_bytes.argtypes = [ctypes.c_int, dp, i32, i32, i64]
    lib.sgqa_status_string.restype = ctypes.c_char_p
    lib.sgqa_status_string.argtypes = [ctypes.c_int]
    lib.sgqa_last_error.restype = ctypes.c_char_p
    lib.sgqa_last_error.argtypes = []
    _lib = lib
    return lib


def check(status: int):
    if status != OK:
        lib = load()
        raise SgqaError(status, f"{lib.sgqa_status_string(status).decode()}: "
                                f"{lib.sgqa_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref: torch.Tensor):
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libsgqa takes device tensors")


def workspace_bytes(op: int, shape: LayerShape, nseq: int, T: int, Lmax: int) -> int:
    d = Dims.of(shape)
    return int(load().sgqa_workspace_bytes(op, ctypes.byref(d), nseq, T, Lmax))


def index_build(shape: LayerShape, kp: torch.Tensor, kb: torch.Tensor, seq_lens,
                blk_begin: int = 0, blk_end: int = -1, stream=None):
    """kp [nseq, Lmax, P] (or [L, P]) -> kb [nseq, nblk, P] (or [nblk, P]), bf16."""
    _need_cuda(kp, kb)
    kp3 = kp if kp.dim() == 3 else kp.unsqueeze(0)
    kb3 = kb if kb.dim() == 3 else kb.unsqueeze(0)
    d = Dims.of(shape)
    seq_lens = list(seq_lens)
    check(load().sgqa_index_build(ctypes.byref(d), _ptr(kp3), kp3.stride(0), _ptr(kb3),
                                  kb3.stride(0), _i64_array(seq_lens), len(seq_lens), blk_begin,
                                  blk_end, _stream(stream, kp)))


def index_build_from_keys(shape: LayerShape, k_cache: torch.Tensor, w_kt: torch.Tensor,
                          kb: torch.Tensor, seq_lens, blk_begin: int = 0, blk_end: int = -1,
                          stream=None):
    """k_cache [nseq, Lmax, Hkv, d] (or [L, Hkv, d]), w_kt [P, Hkv*d] -> kb [nseq, nblk, P]
    (or [nblk, P]), bf16: each block's mean concatenated key, projected."""
    _need_cuda(k_cache, w_kt, kb)
    k4 = k_cache if k_cache.dim() == 4 else k_cache.unsqueeze(0)
    kb3 = kb if kb.dim() == 3 else kb.unsqueeze(0)
    d = Dims.of(shape)
    seq_lens = list(seq_lens)
    check(load().sgqa_index_build_from_keys(ctypes.byref(d), _ptr(k4), k4.stride(0), _ptr(w_kt),
                                            _ptr(kb3), kb3.stride(0), _i64_array(seq_lens),
                                            len(seq_lens), blk_begin, blk_end,
                                            _stream(stream, k_cache)))


def indexer_topk(shape: LayerShape, qp: torch.Tensor, kb: torch.Tensor, q_start, idx: torch.Tensor,
                 sel_scores: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None):
    """qp [nseq, T, P] (or [T, P]), kb [nseq, nblk, P] -> idx [nseq, T, k] int32."""
    _need_cuda(qp, kb, idx, sel_scores, workspace)
    qp3 = qp if qp.dim() == 3 else qp.unsqueeze(0)
    kb3 = kb if kb.dim() == 3 else kb.unsqueeze(0)
    q_start = list(q_start)
    nseq, T = qp3.shape[0], qp3.shape[1]
    if workspace is None:
        lmax = max(q_start) + T
        workspace = torch.empty(workspace_bytes(OP_INDEXER_TOPK, shape, nseq, T, lmax),
                                dtype=torch.uint8, device=qp.device)
    d = Dims.of(shape)
    check(load().sgqa_indexer_topk(ctypes.byref(d), _ptr(qp3), qp3.stride(0), _ptr(kb3),
                                   kb3.stride(0), _i64_array(q_start), nseq, T, _ptr(idx),
                                   _ptr(sel_scores), _ptr(workspace), workspace.numel(),
                                   _stream(stream, qp)))


def sparse_attn_prefill(shape: LayerShape, q, k_cache, v_cache, gate, idx, q_start: int, L: int,
                        softmax_scale: float, out, lse=None, workspace=None, stream=None):
    """Sparse attention for q [T, Hq, d]; ``workspace`` (optional, uint8 device tensor) enables
    the history-sliced launches."""
    _need_cuda(q, k_cache, v_cache, gate, idx, out, lse, workspace)
    d = Dims.of(shape)
    ws_bytes = workspace.numel() if workspace is not None else 0
    check(load().sgqa_sparse_attn_prefill(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(gate), _ptr(idx), q_start, q.shape[0], L,
                                          softmax_scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                          ws_bytes, _stream(stream, q)))


def sparse_attn_decode(shape: LayerShape, q, k_cache, v_cache, gate, idx, cache_lens,
                       softmax_scale: float, out, lse=None, workspace=None, stream=None):
    """q [nseq, Hq, d]; caches [nseq, Lmax, Hkv, d]; idx [nseq, k]; one query per sequence."""
    _need_cuda(q, k_cache, v_cache, gate, idx, out, lse, workspace)
    cache_lens = list(cache_lens)
    nseq = len(cache_lens)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_ATTN_DECODE, shape, nseq, 1, max(cache_lens)),
                                dtype=torch.uint8, device=q.device)
    d = Dims.of(shape)
    check(load().sgqa_sparse_attn_decode(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         k_cache.stride(0), _ptr(gate), _ptr(idx),
                                         _i64_array(cache_lens), nseq, softmax_scale, _ptr(out),
                                         _ptr(lse), _ptr(workspace), workspace.numel(),
                                         _stream(stream, q)))


def sparse_attn_decode_noalloc(shape: LayerShape, q, k_cache, v_cache, gate, idx, cache_lens,
                               softmax_scale: float, out, lse=None, stream=None):
    """sparse_attn_decode without a workspace: the library's fixed per-device scratch holds
    the partial states (calls that overlap on one GPU race)."""
    _need_cuda(q, k_cache, v_cache, gate, idx, out, lse)
    cache_lens = list(cache_lens)
    d = Dims.of(shape)
    check(load().sgqa_sparse_attn_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(k_cache),
                                                 _ptr(v_cache), k_cache.stride(0), _ptr(gate),
                                                 _ptr(idx), _i64_array(cache_lens),
                                                 len(cache_lens), softmax_scale, _ptr(out),
                                                 _ptr(lse), _stream(stream, q)))


def swa_prefill(shape: LayerShape, q, k_cache, v_cache, gate, q_start: int, L: int, window: int,
                softmax_scale: float, out, lse=None, stream=None):
    """Gated sliding-window attention of q [T, Hq, d] over the last `window` positions."""
    _need_cuda(q, k_cache, v_cache, gate, out, lse)
    d = Dims.of(shape)
    check(load().sgqa_swa_prefill(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(gate), q_start, q.shape[0], L, window, softmax_scale,
                                  _ptr(out), _ptr(lse), _stream(stream, q)))


def quantize_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    """FP8 (E4M3) storage of rows: x [..., cols] bf16 -> codes [..., cols] uint8 and one fp32
    scale per row, scales [...]."""
    _need_cuda(x, codes, scales)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if codes.shape != x.shape or scales.numel() != rows:
        raise ValueError("codes must match x and scales hold one value per row")
    check(load().sgqa_quantize_fp8(_ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                   _stream(stream, x)))


def indexer_topk_fp8(shape: LayerShape, qp: torch.Tensor, kb_codes: torch.Tensor,
                     kb_scales: torch.Tensor, q_pos, idx: torch.Tensor,
                     sel_scores: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None):
    """One query per sequence on an FP8 index: qp [nseq, P], kb_codes [nseq, nblk, P] uint8,
    kb_scales [nseq, nblk] fp32 -> idx [nseq, k]."""
    _need_cuda(qp, kb_codes, kb_scales, idx, sel_scores, workspace)
    q_pos = list(q_pos)
    nseq = len(q_pos)
    qp2 = qp.reshape(nseq, -1)
    if (kb_codes.dim() != 3 or kb_scales.shape != kb_codes.shape[:2] or
            not kb_codes.is_contiguous() or not kb_scales.is_contiguous()):
        raise ValueError("FP8 index must be contiguous codes [nseq, nblk, P] with scales "
                         "[nseq, nblk]")
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_INDEXER_TOPK, shape, nseq, 1, max(q_pos) + 1),
                                dtype=torch.uint8, device=qp.device)
    d = Dims.of(shape)
    check(load().sgqa_indexer_topk_fp8(ctypes.byref(d), _ptr(qp2), qp2.stride(0), _ptr(kb_codes),
                                       _ptr(kb_scales), kb_scales.stride(0), _i64_array(q_pos),
                                       nseq, _ptr(idx), _ptr(sel_scores), _ptr(workspace),
                                       workspace.numel(), _stream(stream, qp)))


def sparse_attn_decode_fp8(shape: LayerShape, q, k_codes, v_codes, k_scales, v_scales, gate, idx,
                           cache_lens, softmax_scale: float, out, lse=None, workspace=None,
                           stream=None):
    """q [nseq, Hq, d]; k/v codes [nseq, Lmax, Hkv, d] uint8; k/v scales [nseq, Lmax, Hkv] fp32."""
    _need_cuda(q, k_codes, v_codes, k_scales, v_scales, gate, idx, out, lse, workspace)
    cache_lens = list(cache_lens)
    nseq = len(cache_lens)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_ATTN_DECODE, shape, nseq, 1, max(cache_lens)),
                                dtype=torch.uint8, device=q.device)
    # tokens per sequence slot, the same for codes [nseq, Lmax, Hkv, d] and scales
    # [nseq, Lmax, Hkv] (the ABI takes this count, not an element stride)
    hkv, hd = shape.num_kv_heads, shape.head_dim
    slot = k_codes.shape[1]
    for c_, s_ in ((k_codes, k_scales), (v_codes, v_scales)):
        if (c_.dim() != 4 or c_.shape[1:] != (slot, hkv, hd) or not c_.is_contiguous()
                or s_.shape != c_.shape[:3] or not s_.is_contiguous()):
            raise ValueError("FP8 caches must be contiguous codes [nseq, Lmax, Hkv, d] with "
                             "scales [nseq, Lmax, Hkv]")
    d = Dims.of(shape)
    check(load().sgqa_sparse_attn_decode_fp8(ctypes.byref(d), _ptr(q), _ptr(k_codes),
                                             _ptr(v_codes), _ptr(k_scales), _ptr(v_scales),
                                             slot, _ptr(gate), _ptr(idx),
                                             _i64_array(cache_lens), nseq, softmax_scale,
                                             _ptr(out), _ptr(lse), _ptr(workspace),
                                             workspace.numel(), _stream(stream, q)))


def sparse_attn_backward(shape: LayerShape, q, k_cache, v_cache, gate, idx, q_start: int, L: int,
                         softmax_scale: float, lse, dout, dq, dk, dv, dgate, workspace=None,
                         stream=None, dkdv_row_slice: int = 0, out=None):
    """Backward of sparse_attn_prefill with idx fixed: fp32 dq [T, Hq, d], dk / dv [L, Hkv, d]
    and dgate [T, Hq] from dout [T, Hq, d] and the forward's lse.  ``dkdv_row_slice``: query
    rows per dk / dv phase or slice (0 = chosen by the library; else a multiple of 32); the
    results do not depend on it.  ``out``: the
    forward's output [T, Hq, d]; given, D = dout . out and dq sweeps the selection once."""
    _need_cuda(q, k_cache, v_cache, gate, idx, lse, dout, dq, dk, dv, dgate, workspace, out)
    T = q.shape[0]
    if workspace is None:
        workspace = torch.empty(workspace_bytes(OP_ATTN_BACKWARD, shape, 1, T, L),
                                dtype=torch.uint8, device=q.device)
    d = Dims.of(shape)
    check(load().sgqa_sparse_attn_backward(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(gate), _ptr(idx), q_start, T, L, softmax_scale,
                                           _ptr(lse), _ptr(dout), _ptr(out), _ptr(dq), _ptr(dk),
                                           _ptr(dv), _ptr(dgate), _ptr(workspace),
                                           workspace.numel(), dkdv_row_slice,
                                           _stream(stream, q)))
