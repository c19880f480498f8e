"""fp64 CPU oracle for the Sparse GQA full-attention layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does.

The arithmetic lives in ``sgqa_oracle.c`` (plain C, fp64, OpenMP over query
rows, built with gcc).  This module only marshals numpy arrays into it and
compiles it when no built copy exists.  bf16 tensors travel as their raw
``uint16`` bit patterns and are widened exactly inside the C code.

Each function names the passage of the Step 5 Preview pages it follows; the
readings taken where the pages are silent are listed in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) into ``out``."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", *extra_flags,
               "-o", out + ".tmp", src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    p = ctypes.c_void_p
    lib.orc_num_threads.restype = i32
    lib.orc_num_threads.argtypes = []
    lib.orc_num_blocks.restype = i64
    lib.orc_num_blocks.argtypes = [i64, i32]
    lib.orc_num_candidates.restype = i64
    lib.orc_num_candidates.argtypes = [i64, i32]
    lib.orc_index_build.restype = None
    lib.orc_index_build.argtypes = [p, i64, i32, i32, p]
    lib.orc_index_build_from_keys.restype = None
    lib.orc_index_build_from_keys.argtypes = [p, i64, i32, p, i32, i32, p]
    lib.orc_scores.restype = None
    lib.orc_scores.argtypes = [p, i64, p, i32, i32, p, p, i64]
    lib.orc_topk.restype = None
    lib.orc_topk.argtypes = [p, i64, i64, p, i32, i32, p]
    lib.orc_token_set.restype = i64
    lib.orc_token_set.argtypes = [p, i32, i32, i64, p]
    lib.orc_attend.restype = None
    lib.orc_attend.argtypes = [p, p, p, i64, p, i32, i32, i32, dbl, p, p]
    lib.orc_attend_f64.restype = None
    lib.orc_attend_f64.argtypes = [p, p, p, i64, p, i32, i32, i32, dbl, p, p]
    lib.orc_attend_backward.restype = None
    lib.orc_attend_backward.argtypes = [p, p, p, i64, p, p, i32, i32, i32, dbl, p, p, p, p]
    lib.orc_sparse_attention_backward.restype = ctypes.c_int
    lib.orc_sparse_attention_backward.argtypes = [p, p, i64, p, p, i64, p, p, i32, i32, i32, i32,
                                                  i32, dbl, p, p, p, p, p]
    lib.orc_e4m3_decode.restype = dbl
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_quantize_rows.restype = None
    lib.orc_quantize_rows.argtypes = [p, i64, i32, p, p]
    lib.orc_dequant_rows.restype = None
    lib.orc_dequant_rows.argtypes = [p, p, i64, i32, p]
    lib.orc_window_token_set.restype = i64
    lib.orc_window_token_set.argtypes = [i64, i64, p]
    lib.orc_window_attention.restype = ctypes.c_int
    lib.orc_window_attention.argtypes = [p, p, i64, p, p, i64, p, i64, i32, i32, i32, dbl, p, p]
    lib.orc_sparse_attention.restype = ctypes.c_int
    lib.orc_sparse_attention.argtypes = [p, p, i64, p, p, i64, p, p, i32, i32, i32, i32, i32,
                                         dbl, p, p]
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected raw bf16 bits as uint16, got {a.dtype}")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads(lib=None) -> int:
    """Threads the oracle's parallel loops run on."""
    return int((lib or load()).orc_num_threads())


def num_blocks(L: int, B: int, lib=None) -> int:
    return int((lib or load()).orc_num_blocks(L, B))


def num_candidates(t: int, B: int, lib=None) -> int:
    return int((lib or load()).orc_num_candidates(t, B))


def index_build(kp_bits: np.ndarray, B: int, lib=None) -> np.ndarray:
    """Block compression: mean of the proxy keys over each block of B tokens.

    Follows ai4snews Interpretation para. 2 (indexer entries of neighbouring
    positions compressed into blocks of 8) with the mean as the block
    representation.  ``kp_bits``: [L, P] uint16 -> [ceil(L/B), P] float64.
    """
    lib = lib or load()
    kp = _u16(kp_bits)
    L, P = kp.shape
    kb = np.empty((num_blocks(L, B, lib), P), dtype=np.float64)
    lib.orc_index_build(_ptr(kp), L, P, B, _ptr(kb))
    return kb


def index_build_from_keys(k_bits: np.ndarray, wt_bits: np.ndarray, B: int, lib=None) -> np.ndarray:
    """Block representations from the keys: the projection (``wt`` = W transposed, [P, width])
    of each block's mean concatenated key, which equals the block mean of the projected keys
    (the proxy width is fixed by phantomic12 config.json / sparse_config; blocks of 8 by
    ai4snews Interpretation para. 2).  ``k_bits``: [L, Hkv, d] or [L, width] uint16 ->
    [ceil(L/B), P] float64."""
    lib = lib or load()
    K = _u16(k_bits)
    L = K.shape[0]
    K = K.reshape(L, -1)
    wt = _u16(wt_bits)
    P, width = wt.shape
    if K.shape[1] != width:
        raise ValueError("key width does not match the projection")
    kb = np.empty((num_blocks(L, B, lib), P), dtype=np.float64)
    lib.orc_index_build_from_keys(_ptr(K), L, width, _ptr(wt), P, B, _ptr(kb))
    return kb


def scores(qp_bits: np.ndarray, t: np.ndarray, B: int, kb: np.ndarray, width: int | None = None,
           lib=None) -> np.ndarray:
    """Indexer scores qp[t] . kb[j] for j < floor(t/B) (phantomic12 sparse_config).

    ``qp_bits``: [n, P] uint16; ``t``: [n] positions; ``kb``: [nblk, P] float64.
    Returns [n, width] float64; entries at or beyond a row's candidate count are NaN.
    """
    lib = lib or load()
    qp = _u16(qp_bits)
    t = np.ascontiguousarray(t, dtype=np.int64)
    kb = np.ascontiguousarray(kb, dtype=np.float64)
    n, P = qp.shape
    if width is None:
        width = max(1, int(t.max()) // B) if n else 1
    out = np.full((n, width), np.nan, dtype=np.float64)
    if n and int(t.max()) // B > width:
        raise ValueError("width smaller than the largest candidate count")
    if n and int(t.max()) // B > kb.shape[0]:
        raise ValueError("kb has fewer rows than the candidates need")
    lib.orc_scores(_ptr(qp), n, _ptr(t), B, P, _ptr(kb), _ptr(out), width)
    return out


def topk(score_rows: np.ndarray, t: np.ndarray, B: int, k: int, lib=None) -> np.ndarray:
    """Causal top-k by explicit sort with the own block forced (int32 [n, k], asc, -1 pad)."""
    lib = lib or load()
    s = np.ascontiguousarray(score_rows, dtype=np.float64)
    t = np.ascontiguousarray(t, dtype=np.int64)
    n = t.shape[0]
    if s.ndim != 2 or s.shape[0] != n:
        raise ValueError("score rows do not match t")
    if n and int(t.max()) // B > s.shape[1]:
        raise ValueError("score rows narrower than the candidate count")
    idx = np.empty((n, k), dtype=np.int32)
    lib.orc_topk(_ptr(s), n, s.shape[1], _ptr(t), B, k, _ptr(idx))
    return idx


def token_set(sel: np.ndarray, B: int, t: int, lib=None) -> np.ndarray:
    """Positions a query at t attends to, given its selected-block row."""
    lib = lib or load()
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    k = sel.shape[0]
    buf = np.empty(max(1, k * B), dtype=np.int64)
    n = lib.orc_token_set(_ptr(sel), k, B, int(t), _ptr(buf))
    return buf[:n].copy()


def attend(q_bits, k_rows, v_rows, gate_bits, scale: float, lib=None):
    """Gated GQA of one query over explicit K/V rows -> (out [Hq, d], lse [Hq])."""
    lib = lib or load()
    q = _u16(q_bits)
    kr = _u16(k_rows)
    vr = _u16(v_rows)
    g = _u16(gate_bits)
    Hq, d = q.shape
    n, Hkv, d2 = kr.shape
    if d2 != d or vr.shape != kr.shape or g.shape != (Hq,) or Hq % Hkv:
        raise ValueError("shape mismatch in attend")
    out = np.empty((Hq, d), dtype=np.float64)
    lse = np.empty((Hq,), dtype=np.float64)
    lib.orc_attend(_ptr(q), _ptr(kr), _ptr(vr), n, _ptr(g), Hq, Hkv, d, float(scale), _ptr(out),
                   _ptr(lse))
    return out, lse


def attend_f64(q_bits, k_rows, v_rows, gate_bits, scale: float, lib=None):
    """Gated GQA of one query over explicit K/V rows given as float64 [n, Hkv, d] (for
    dequantised FP8 rows) -> (out [Hq, d], lse [Hq])."""
    lib = lib or load()
    q = _u16(q_bits)
    kr = np.ascontiguousarray(k_rows, dtype=np.float64)
    vr = np.ascontiguousarray(v_rows, dtype=np.float64)
    g = _u16(gate_bits)
    Hq, d = q.shape
    n, Hkv, d2 = kr.shape
    if d2 != d or vr.shape != kr.shape or g.shape != (Hq,) or Hq % Hkv:
        raise ValueError("shape mismatch in attend_f64")
    out = np.empty((Hq, d), dtype=np.float64)
    lse = np.empty((Hq,), dtype=np.float64)
    lib.orc_attend_f64(_ptr(q), _ptr(kr), _ptr(vr), n, _ptr(g), Hq, Hkv, d, float(scale),
                       _ptr(out), _ptr(lse))
    return out, lse


def e4m3_decode(codes, lib=None) -> np.ndarray:
    """OCP E4M3 codes -> float64 values (NaN for the NaN codes)."""
    lib = lib or load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_e4m3_decode(int(x)) for x in c], dtype=np.float64).reshape(
        np.shape(codes))


def e4m3_encode(values, lib=None) -> np.ndarray:
    """float32 values -> nearest E4M3 codes (ties to even, saturating at +-448)."""
    lib = lib or load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.orc_e4m3_encode(float(x)) for x in v], dtype=np.uint8).reshape(
        np.shape(values))


def quantize_rows(x_bits: np.ndarray, lib=None):
    """FP8 storage of cached rows: bf16 bits [..., cols] -> (e4m3 codes uint8 [..., cols],
    fp32 scales [...]); one scale per row, amax / 448, all in fp32 (see the C header)."""
    lib = lib or load()
    x = _u16(x_bits)
    cols = x.shape[-1]
    rows = x.size // cols if cols else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib.orc_quantize_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scales))
    return codes, scales


def dequant_rows(codes: np.ndarray, scales: np.ndarray, lib=None) -> np.ndarray:
    """e4m3 codes [..., cols] and fp32 scales [...] -> float64 values."""
    lib = lib or load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    cols = c.shape[-1]
    rows = c.size // cols if cols else 0
    if sc.size != rows:
        raise ValueError("one scale per row")
    out = np.empty(c.shape, dtype=np.float64)
    lib.orc_dequant_rows(_ptr(c), _ptr(sc), rows, cols, _ptr(out))
    return out


def sparse_attention(q_bits, t, K_bits, V_bits, G_bits, idx, B: int, scale: float, lib=None):
    """Sparse gated GQA for query rows at positions ``t`` with the cache on the host.

    ``q_bits`` [n, Hq, d], ``K_bits``/``V_bits`` [L, Hkv, d], ``G_bits`` [n, Hq],
    ``idx`` [n, k] int32.  Returns (out [n, Hq, d] float64, lse [n, Hq] float64).
    """
    lib = lib or load()
    q = _u16(q_bits)
    K = _u16(K_bits)
    V = _u16(V_bits)
    G = _u16(G_bits)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    t = np.ascontiguousarray(t, dtype=np.int64)
    n, Hq, d = q.shape
    L, Hkv, d2 = K.shape
    if d2 != d or V.shape != K.shape or G.shape != (n, Hq) or idx.shape[0] != n or t.shape != (n,):
        raise ValueError("shape mismatch in sparse_attention")
    k = idx.shape[1]
    out = np.empty((n, Hq, d), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    rc = lib.orc_sparse_attention(_ptr(q), _ptr(t), n, _ptr(K), _ptr(V), L, _ptr(G), _ptr(idx), k,
                                  B, Hq, Hkv, d, float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("a selected token lies outside the cache")
    return out, lse


def sparse_attention_backward(q_bits, t, K_bits, V_bits, G_bits, idx, B: int, scale: float,
                              gout_bits, lib=None):
    """Backward of sparse_attention with the selection fixed, for the loss whose gradient
    with respect to out is ``gout_bits`` [n, Hq, d] (bf16 bits).  Returns (dq [n, Hq, d],
    dK [L, Hkv, d], dV [L, Hkv, d], dgate [n, Hq]), all float64; dK / dV sum over the rows."""
    lib = lib or load()
    q = _u16(q_bits)
    K = _u16(K_bits)
    V = _u16(V_bits)
    G = _u16(G_bits)
    go = _u16(gout_bits)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    t = np.ascontiguousarray(t, dtype=np.int64)
    n, Hq, d = q.shape
    L, Hkv, d2 = K.shape
    if (d2 != d or V.shape != K.shape or G.shape != (n, Hq) or idx.shape[0] != n
            or t.shape != (n,) or go.shape != q.shape):
        raise ValueError("shape mismatch in sparse_attention_backward")
    k = idx.shape[1]
    dq = np.empty((n, Hq, d), dtype=np.float64)
    dK = np.empty((L, Hkv, d), dtype=np.float64)
    dV = np.empty((L, Hkv, d), dtype=np.float64)
    dg = np.empty((n, Hq), dtype=np.float64)
    rc = lib.orc_sparse_attention_backward(_ptr(q), _ptr(t), n, _ptr(K), _ptr(V), L, _ptr(G),
                                           _ptr(idx), k, B, Hq, Hkv, d, float(scale), _ptr(go),
                                           _ptr(dq), _ptr(dK), _ptr(dV), _ptr(dg))
    if rc != 0:
        raise ValueError("a selected token lies outside the cache")
    return dq, dK, dV, dg


def window_attention(q_bits, t, K_bits, V_bits, G_bits, window: int, scale: float, lib=None):
    """Gated sliding-window attention (the ``window`` most recent positions, own included)
    for query rows at positions ``t``; shapes as :func:`sparse_attention` without idx."""
    lib = lib or load()
    q = _u16(q_bits)
    K = _u16(K_bits)
    V = _u16(V_bits)
    G = _u16(G_bits)
    t = np.ascontiguousarray(t, dtype=np.int64)
    n, Hq, d = q.shape
    L, Hkv, d2 = K.shape
    if d2 != d or V.shape != K.shape or G.shape != (n, Hq) or t.shape != (n,):
        raise ValueError("shape mismatch in window_attention")
    out = np.empty((n, Hq, d), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    rc = lib.orc_window_attention(_ptr(q), _ptr(t), n, _ptr(K), _ptr(V), L, _ptr(G), int(window),
                                  Hq, Hkv, d, float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("a window position lies outside the cache")
    return out, lse
