"""The C-ABI library loads, exports every symbol the header declares, and rejects bad
arguments in host code before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_sparse_18_amd import REAL, TINY, probe, sgqa
from long_context_sparse_18_amd.configs import with_selection

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgqa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "sgqa_probe.h")

FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sgqa.load()
    names = declared_functions()
    assert set(names) == set(sgqa.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_symbol():
    """The machine-peak probes live in libsgqa_probe.so, beside the layer's library, which
    exports none of them."""
    lib = probe.load()
    names = declared_functions(PROBE_HEADER)
    assert set(names) == set(probe.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    for n in names:
        assert not hasattr(sgqa.load(), n), n


def test_status_strings():
    lib = sgqa.load()
    for st in range(6):
        assert lib.sgqa_status_string(st)
    assert lib.sgqa_status_string(99) == b"unknown status"


def dims(**kw):
    s = sgqa.Dims.of(REAL)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def call_prefill(d, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, idx=FAKE, q_start=0, T=16, L=16, scale=0.07, out=FAKE,
             lse=None)
    a.update(kw)
    return sgqa.load().sgqa_sparse_attn_prefill(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"],
                                                a["idx"], a["q_start"], a["T"], a["L"], a["scale"],
                                                a["out"], a["lse"], a.get("ws"), a.get("wsb", 0),
                                                None)


@pytest.mark.parametrize("kw,want", [
    (dict(num_kv_heads=3), sgqa.ERR_SHAPE),           # 64 % 3 != 0
    (dict(num_kv_heads=2), sgqa.ERR_UNSUPPORTED),     # 32 heads per group
    (dict(head_dim=96), sgqa.ERR_UNSUPPORTED),
    (dict(head_dim=0), sgqa.ERR_SHAPE),
    (dict(block_size=3), sgqa.ERR_UNSUPPORTED),
    (dict(block_size=0), sgqa.ERR_SHAPE),
    (dict(topk_blocks=0), sgqa.ERR_SHAPE),
    (dict(topk_blocks=4097), sgqa.ERR_UNSUPPORTED),
    (dict(topk_blocks=2048, block_size=32), sgqa.ERR_UNSUPPORTED),  # 65536 tokens
])
def test_prefill_rejects_bad_dims(kw, want):
    assert call_prefill(dims(**kw)) == want


def test_prefill_rejects_bad_sizes_and_pointers():
    d = dims()
    assert call_prefill(d, q_start=10, T=16, L=20) == sgqa.ERR_SHAPE
    assert call_prefill(d, T=-1) == sgqa.ERR_SHAPE
    assert call_prefill(d, q=None) == sgqa.ERR_NULL
    assert call_prefill(d, out=None) == sgqa.ERR_NULL
    assert call_prefill(d, q=ctypes.c_void_p((1 << 20) + 2)) == sgqa.ERR_SHAPE  # misaligned
    assert call_prefill(d, scale=float("inf")) == sgqa.ERR_SHAPE
    assert call_prefill(d, ws=FAKE, wsb=100) == sgqa.ERR_WORKSPACE
    assert call_prefill(d, ws=ctypes.c_void_p((1 << 20) + 8), wsb=1 << 30) == sgqa.ERR_SHAPE
    assert call_prefill(d, T=0) == sgqa.OK  # nothing to do, no HIP call
    assert sgqa.load().sgqa_last_error() == b""
    assert call_prefill(d, q_start=10, T=16, L=20) == sgqa.ERR_SHAPE
    assert b"exceeds L" in sgqa.load().sgqa_last_error()
    # more query rows than one call takes (the launches would pass 32-bit work-item counts)
    big = (1 << 24) + 1
    assert call_prefill(d, T=big, L=big) == sgqa.ERR_UNSUPPORTED
    assert b"per call" in sgqa.load().sgqa_last_error()
    assert call_prefill(d, T=1 << 24, L=1 << 24, q=None) == sgqa.ERR_NULL  # the limit itself is fine


def test_null_dims():
    lib = sgqa.load()
    assert lib.sgqa_sparse_attn_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 0.1, FAKE,
                                        None, None, 0, None) == sgqa.ERR_NULL


def test_indexer_validation():
    lib = sgqa.load()
    d = dims()
    qs = (ctypes.c_int64 * 2)(0, 0)

    def call(qp=FAKE, kb=FAKE, q_start=qs, nseq=1, T=64, idx=FAKE, ws=FAKE, wsb=1 << 30,
             qp_stride=64 * 256, d=d):
        return lib.sgqa_indexer_topk(ctypes.byref(d), qp, qp_stride, kb, 1 << 20, q_start, nseq, T,
                                     idx, None, ws, wsb, None)

    assert call(qp=None) == sgqa.ERR_NULL
    assert call(idx=None) == sgqa.ERR_NULL
    assert call(q_start=None) == sgqa.ERR_NULL
    assert call(T=-1) == sgqa.ERR_SHAPE
    assert call(nseq=65) == sgqa.ERR_UNSUPPORTED
    assert call(ws=None) == sgqa.ERR_WORKSPACE
    assert call(wsb=16) == sgqa.ERR_WORKSPACE
    assert call(nseq=2, qp_stride=100) == sgqa.ERR_SHAPE
    neg = (ctypes.c_int64 * 1)(-5)
    assert call(q_start=neg) == sgqa.ERR_SHAPE
    bad = dims(proxy_dim=48)
    assert call(d=bad) == sgqa.ERR_UNSUPPORTED
    assert call(T=0) == sgqa.OK


def test_index_build_validation():
    lib = sgqa.load()
    d = dims()
    lens = (ctypes.c_int64 * 2)(1024, 1024)
    assert lib.sgqa_index_build(ctypes.byref(d), None, 0, FAKE, 0, lens, 1, 0, -1, None) == sgqa.ERR_NULL
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 0, FAKE, 0, None, 1, 0, -1, None) == sgqa.ERR_NULL
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 0, FAKE, 0, lens, 1, -1, -1, None) == sgqa.ERR_SHAPE
    # two sequences need strides that separate them
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 10, FAKE, 1 << 20, lens, 2, 0, -1, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 1 << 20, FAKE, 8, lens, 2, 0, -1, None) == sgqa.ERR_SHAPE
    neg = (ctypes.c_int64 * 1)(-1)
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 0, FAKE, 0, neg, 1, 0, -1, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_index_build(ctypes.byref(d), FAKE, 0, FAKE, 0, lens, 0, 0, -1, None) == sgqa.OK


def test_index_build_from_keys_validation():
    lib = sgqa.load()
    lens = (ctypes.c_int64 * 2)(1024, 1024)
    width = REAL.num_kv_heads * REAL.head_dim

    def call(d=None, k=FAKE, wt=FAKE, kb=FAKE, kstride=1024 * width, kbstride=128 * 256,
             lens=lens, nseq=2, b0=0):
        d = d or dims()
        return lib.sgqa_index_build_from_keys(ctypes.byref(d), k, kstride, wt, kb, kbstride, lens,
                                              nseq, b0, -1, None)

    assert call(k=None) == sgqa.ERR_NULL
    assert call(wt=None) == sgqa.ERR_NULL
    assert call(lens=None) == sgqa.ERR_NULL
    assert call(b0=-1) == sgqa.ERR_SHAPE
    assert call(kstride=10) == sgqa.ERR_SHAPE
    assert call(kbstride=8) == sgqa.ERR_SHAPE
    assert call(wt=ctypes.c_void_p((1 << 20) + 2)) == sgqa.ERR_SHAPE
    assert call(d=dims(proxy_dim=96)) == sgqa.ERR_UNSUPPORTED
    assert call(d=dims(head_dim=96)) == sgqa.ERR_UNSUPPORTED
    assert call(nseq=65) == sgqa.ERR_UNSUPPORTED
    assert call(nseq=0) == sgqa.OK


def test_fp8_validation():
    lib = sgqa.load()
    u8 = FAKE
    assert lib.sgqa_quantize_fp8(FAKE, 10, 0, u8, FAKE, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_quantize_fp8(FAKE, -1, 8, u8, FAKE, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_quantize_fp8(FAKE, 10, 5000, u8, FAKE, None) == sgqa.ERR_UNSUPPORTED
    assert lib.sgqa_quantize_fp8(None, 10, 8, u8, FAKE, None) == sgqa.ERR_NULL
    assert lib.sgqa_quantize_fp8(FAKE, 0, 8, u8, FAKE, None) == sgqa.OK
    d = dims()
    pos = (ctypes.c_int64 * 2)((1 << 20) - 1, (1 << 20) - 1)
    need = lib.sgqa_workspace_bytes(sgqa.OP_INDEXER_TOPK, ctypes.byref(d), 2, 1, 1 << 20)

    def topk(d=d, qp=FAKE, ws=FAKE, wsb=need, kbs_stride=1 << 17):
        return lib.sgqa_indexer_topk_fp8(ctypes.byref(d), qp, 256, FAKE, FAKE, kbs_stride, pos, 2,
                                         FAKE, None, ws, wsb, None)

    assert topk(qp=None) == sgqa.ERR_NULL
    assert topk(d=dims(proxy_dim=32)) == sgqa.ERR_UNSUPPORTED
    assert topk(d=dims(topk_blocks=1)) == sgqa.ERR_UNSUPPORTED
    assert topk(wsb=need - 1) == sgqa.ERR_WORKSPACE
    assert topk(kbs_stride=100) == sgqa.ERR_SHAPE
    lens = (ctypes.c_int64 * 2)(1 << 20, 1 << 20)
    dneed = lib.sgqa_workspace_bytes(sgqa.OP_ATTN_DECODE, ctypes.byref(d), 2, 1, 1 << 20)

    def attn(q=FAKE, stride=1 << 20, wsb=dneed, ks=FAKE):
        return lib.sgqa_sparse_attn_decode_fp8(ctypes.byref(d), q, FAKE, FAKE, ks, FAKE, stride,
                                               FAKE, FAKE, lens, 2, 0.07, FAKE, None, FAKE, wsb,
                                               None)

    assert attn(q=None) == sgqa.ERR_NULL
    assert attn(ks=None) == sgqa.ERR_NULL
    assert attn(stride=100) == sgqa.ERR_SHAPE
    assert attn(wsb=dneed - 1) == sgqa.ERR_WORKSPACE


def test_backward_validation():
    lib = sgqa.load()
    d = dims()
    need = lib.sgqa_workspace_bytes(sgqa.OP_ATTN_BACKWARD, ctypes.byref(d), 1, 64, 1024)
    assert need > 0

    def call(q=FAKE, lse=FAKE, T=64, L=1024, q_start=0, ws=FAKE, wsb=need, slice_=0):
        return lib.sgqa_sparse_attn_backward(ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, q_start, T,
                                             L, 0.07, lse, FAKE, None, FAKE, FAKE, FAKE, FAKE, ws,
                                             wsb,
                                             slice_, None)

    assert call(q=None) == sgqa.ERR_NULL
    assert call(lse=None) == sgqa.ERR_NULL
    assert call(q_start=1000) == sgqa.ERR_SHAPE   # rows past the cache
    assert call(T=-1) == sgqa.ERR_SHAPE
    assert call(wsb=need - 1) == sgqa.ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16)) == sgqa.ERR_SHAPE
    assert call(T=(1 << 24) + 1, L=(1 << 24) + 1) == sgqa.ERR_UNSUPPORTED
    assert call(T=64, L=((1 << 24) + 1) * 8) == sgqa.ERR_UNSUPPORTED  # cache blocks
    assert call(slice_=16) == sgqa.ERR_SHAPE      # dk / dv row slices are whole bitmap words
    assert call(slice_=-32) == sgqa.ERR_SHAPE
    assert call(T=0) == sgqa.OK
    assert call(T=0, slice_=64) == sgqa.OK
    assert lib.sgqa_workspace_bytes(sgqa.OP_ATTN_BACKWARD, ctypes.byref(d), 2, 64, 1024) == 0


def test_probe_validation():
    lib = probe.load()
    sink = FAKE
    assert lib.sgqa_probe_mfma_bf16(0, 10, sink, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_mfma_bf16(64, 0, sink, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_mfma_bf16(64, 8193, sink, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_mfma_bf16(64, 10, None, None) == sgqa.ERR_NULL
    assert lib.sgqa_probe_read(FAKE, 0, sink, 8, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_read(FAKE, 24, sink, 8, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_read(FAKE, 1024, sink, 0, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_read(FAKE, 1024, sink, 65537, None) == sgqa.ERR_SHAPE
    assert lib.sgqa_probe_read(None, 1024, sink, 8, None) == sgqa.ERR_NULL
    assert lib.sgqa_probe_read(ctypes.c_void_p((1 << 20) + 8), 1024, sink, 8, None) == \
        sgqa.ERR_SHAPE
    g = lib.sgqa_probe_gather
    assert g(FAKE, 0, 384, FAKE, 10, sink, 8, None) == sgqa.ERR_SHAPE
    assert g(FAKE, 100, 392, FAKE, 10, sink, 8, None) == sgqa.ERR_SHAPE
    assert g(FAKE, 100, 65552, FAKE, 10, sink, 8, None) == sgqa.ERR_SHAPE
    assert g(FAKE, 100, 384, FAKE, 0, sink, 8, None) == sgqa.ERR_SHAPE
    assert g(FAKE, 100, 384, FAKE, 10, sink, 0, None) == sgqa.ERR_SHAPE
    assert g(FAKE, 100, 384, None, 10, sink, 8, None) == sgqa.ERR_NULL
    assert g(ctypes.c_void_p((1 << 20) + 8), 100, 384, FAKE, 10, sink, 8, None) == sgqa.ERR_SHAPE
    assert b"aligned" in lib.sgqa_probe_last_error()


def test_decode_validation():
    lib = sgqa.load()
    d = dims()
    lens = (ctypes.c_int64 * 2)(1 << 20, 1 << 20)
    need = lib.sgqa_workspace_bytes(sgqa.OP_ATTN_DECODE, ctypes.byref(d), 2, 1, 1 << 20)
    assert need > 0

    def call(lens=lens, nseq=2, stride=(1 << 20) * 4 * 192, ws=FAKE, wsb=need, q=FAKE):
        return lib.sgqa_sparse_attn_decode(ctypes.byref(d), q, FAKE, FAKE, stride, FAKE, FAKE, lens,
                                           nseq, 0.07, FAKE, None, ws, wsb, None)

    assert call(q=None) == sgqa.ERR_NULL
    assert call(lens=None) == sgqa.ERR_NULL
    assert call(stride=100) == sgqa.ERR_SHAPE
    assert call(wsb=need - 1) == sgqa.ERR_WORKSPACE
    assert call(ws=None) == sgqa.ERR_WORKSPACE
    zero = (ctypes.c_int64 * 1)(0)
    assert call(lens=zero, nseq=1) == sgqa.ERR_SHAPE
    assert call(nseq=65) == sgqa.ERR_UNSUPPORTED
    assert call(nseq=0) == sgqa.OK


def test_decode_noalloc_validation():
    """The decode entry point without a workspace: the same checks, and calls whose partial
    states exceed the library's 16 MiB scratch are refused before any HIP call."""
    lib = sgqa.load()
    lens = (ctypes.c_int64 * 64)(*([1 << 16] * 64))

    def call(d, nseq=2, q=FAKE, lens=lens, stride=(1 << 16) * 4 * 192):
        return lib.sgqa_sparse_attn_decode_noalloc(ctypes.byref(d), q, FAKE, FAKE, stride, FAKE,
                                                   FAKE, lens, nseq, 0.07, FAKE, None, None)

    d = dims()
    assert call(d, q=None) == sgqa.ERR_NULL
    assert call(d, lens=None) == sgqa.ERR_NULL
    assert call(d, stride=100) == sgqa.ERR_SHAPE
    assert call(d, nseq=65) == sgqa.ERR_UNSUPPORTED
    assert call(d, nseq=0) == sgqa.OK
    # 128 heads of d 192 over 64 sequences: 64 x 4 parts x 128 x 195 x 4 B = 25.6 MB > 16 MiB
    big = dims(num_q_heads=128, num_kv_heads=8)
    assert call(big, nseq=64, stride=(1 << 16) * 8 * 192) == sgqa.ERR_UNSUPPORTED
    assert b"scratch" in lib.sgqa_last_error()


def test_workspace_sizes():
    # a 32K prefill in one pass of the path without a score matrix: per row 1024 sample keys,
    # threshold, count, queue slot and a 2048-entry candidate list; 64 fallback score rows of
    # ld = 4096 floats and 256 bytes of counters
    fused = 256 + 64 * 4096 * 4 + 32768 * (1024 * 4 + 12 + 2048 * 8)
    assert sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, REAL, 1, 32768, 32768) == fused
    # capped at 2 GiB for the 128K prefill
    big = sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, REAL, 1, 131072, 131072)
    assert big <= 2 << 30
    # the chunked prefill (131072 candidates: 4096 sample keys, 4096-entry lists) in one pass
    ch = sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, REAL, 1, 8192, 1048580)
    assert ch == 256 + 64 * 131072 * 4 + 8192 * (4096 * 4 + 12 + 4096 * 8)
    # k beyond the selection without a score matrix: whole score rows, 2 GiB at most
    wide = sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, with_selection(REAL, 1, 2048), 1, 32768,
                                32768)
    assert wide == 2 << 30  # 32768 rows x ld 32768 x 4 B = 4 GiB, capped in 64-row passes
    # decode: 32 splits of 16 blocks; partial o + (max, two sums) per (seq, split, head)
    ws = sgqa.workspace_bytes(sgqa.OP_ATTN_DECODE, REAL, 16, 1, 1 << 20)
    assert ws == 16 * 32 * 64 * (192 + 3) * 4
    assert sgqa.workspace_bytes(sgqa.OP_ATTN_DECODE, with_selection(TINY, 8, 16), 1, 1, 1024) > 0
    assert sgqa.workspace_bytes(7, REAL, 1, 1, 1) == 0
    # prefill attention: the parked state of min(T, 32768) rows (4 groups x 64 lanes x 52
    # floats each at d = 192), and at least the resident prefill's progress words (one 4-byte
    # word per resident wave: 256 CUs x 8 workgroups x 4 waves)
    assert sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, REAL, 1, 1, 1 << 17) == 4 * 64 * 52 * 4
    assert sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, REAL, 1, 1 << 17, 1 << 17) == \
        32768 * 4 * 64 * 52 * 4
    assert sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, TINY, 1, 1, 1024) == 256 * 8 * 4 * 4


def test_swa_validation():
    lib = sgqa.load()
    d = dims()

    def call(q=FAKE, T=64, L=1024, q_start=0, window=512, scale=0.07, out=FAKE):
        return lib.sgqa_swa_prefill(ctypes.byref(d), q, FAKE, FAKE, FAKE, q_start, T, L, window,
                                    scale, out, None, None)

    assert call(q=None) == sgqa.ERR_NULL
    assert call(out=None) == sgqa.ERR_NULL
    assert call(window=0) == sgqa.ERR_SHAPE
    assert call(q_start=1000) == sgqa.ERR_SHAPE
    assert call(scale=float("nan")) == sgqa.ERR_SHAPE
    assert call(q=ctypes.c_void_p((1 << 20) + 2)) == sgqa.ERR_SHAPE
    assert call(T=(1 << 24) + 1, L=(1 << 24) + 1) == sgqa.ERR_UNSUPPORTED
    assert call(T=0) == sgqa.OK
