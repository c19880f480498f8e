"""Comparison rules between the HIP path and the oracle (test infrastructure).

Tolerances follow the stated bars for this layer:
  * block-compressed keys within 1e-3 relative -- checked rounding-aware, since a
    bf16 output carries up to half a bf16 ulp of rounding on top of any error:
    |kb_gpu - kb_ref| <= 1e-3 |kb_ref| + ulp_bf16(kb_ref) / 2;
  * indexer scores within 2e-3 relative, relative to the row's largest score:
    |s_gpu - s_ref| <= tau = 2e-3 * max_j |s_ref[j]|;
  * top-k sets equal except inside the tolerance band: a GPU whose scores are
    within tau of the oracle's can swap only blocks whose oracle scores lie in
    [s_(k) - 2 tau, s_(k-1) + 2 tau] (s_(k-1): last kept, s_(k): first dropped),
    so every block in the symmetric difference must lie there; a gap wider than
    2 tau therefore forces identical sets;
  * attention, given identical selections: max-abs error <= 1e-2 (plus half a
    bf16 ulp of the reference value where |o| >= 4) and relative L2 <= 5e-3.
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 2e-3
KB_RTOL = 1e-3
ATTN_MAX_ABS = 1e-2
ATTN_REL_L2 = 5e-3
LSE_ABS = 4e-3


def widen(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.ldexp(1.0, (e - 7).astype(int))


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), through float32."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return widen(u.astype(np.uint16))


def check_kb(kb_gpu_bits: np.ndarray, kb_ref: np.ndarray) -> dict:
    g = widen(kb_gpu_bits)
    err = np.abs(g - kb_ref)
    tol = KB_RTOL * np.abs(kb_ref) + 0.5 * ulp_bf16(kb_ref)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} kb elements out of tolerance; worst "
                           f"{(err - tol).max():.3g} over")
    exact = float(np.mean(g == rne_bf16(kb_ref)))
    return {"kb_bit_equal_to_rne": exact, "kb_max_abs_err": float(err.max())}


def check_kb_projected(kb_gpu_bits: np.ndarray, kb_ref: np.ndarray) -> dict:
    """Block representations formed by a projection (a dot product over Hkv*d terms): the
    error of each element is measured against its row's largest magnitude, as for the
    indexer scores, plus half a bf16 ulp of the element for the final rounding."""
    g = widen(kb_gpu_bits)
    err = np.abs(g - kb_ref)
    scale = np.abs(kb_ref).max(axis=-1, keepdims=True)
    tol = KB_RTOL * scale + 0.5 * ulp_bf16(kb_ref)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} kb elements out of tolerance; worst "
                           f"{(err - tol).max():.3g} over")
    exact = float(np.mean(g == rne_bf16(kb_ref)))
    return {"kb_bit_equal_to_rne": exact, "kb_max_abs_err": float(err.max()),
            "kb_max_rel_to_row": float((err / scale).max())}


def score_tau(ref_row: np.ndarray) -> float:
    return SCORE_RTOL * float(np.max(np.abs(ref_row))) if ref_row.size else 0.0


def check_selection(idx_row: np.ndarray, ref_scores: np.ndarray, c: int, k: int,
                    ref_idx_row: np.ndarray, end_to_end: bool = False) -> bool:
    """Validate one GPU selection row against the oracle's scores and selection.

    Stage-isolated (the oracle scored the GPU's own bf16 index): the sets must be identical
    whenever the (k-1)-th and k-th past-block scores are more than tau apart, and otherwise
    differ only in blocks within tau of that boundary.  End to end (the oracle scored its own
    fp64 index): the GPU's scores carry the bf16 rounding of the index, up to tau each, so two
    blocks up to 2 tau apart can trade places; the same rule then holds with 2 tau.
    Returns True when the sets are identical, False when they differ only inside the band;
    raises AssertionError otherwise."""
    row = np.asarray(idx_row)
    n = min(k, c + 1)
    valid = row[:n]
    assert np.all(row[n:] == -1), f"padding wrong: {row[n:][:8]}"
    assert np.all(np.diff(valid) > 0), "not strictly ascending"
    assert valid[-1] == c, f"own block {c} missing (last {valid[-1]})"
    assert valid.min() >= 0 and valid.max() <= c
    if c <= k - 1:
        assert np.array_equal(valid, np.arange(c + 1))
        return True
    G = set(valid[:-1].tolist())
    R = set(np.asarray(ref_idx_row)[: k - 1].tolist())
    if G == R:
        return True
    s = ref_scores[:c]
    order = np.lexsort((np.arange(c), -s))
    s_keep, s_drop = s[order[k - 2]], s[order[k - 1]]
    tau = score_tau(s) * (2.0 if end_to_end else 1.0)
    assert s_keep - s_drop <= tau, (f"selection differs although the boundary gap "
                                    f"{s_keep - s_drop:.6g} exceeds the band {tau:.6g}")
    lo, hi = s_drop - tau, s_keep + tau
    diff = np.array(sorted(G ^ R))
    out = diff[(s[diff] < lo) | (s[diff] > hi)]
    assert out.size == 0, (f"selection differs outside the band: blocks {out[:8]} scores "
                           f"{s[out[:8]]} band [{lo:.6g}, {hi:.6g}]")
    return False


def check_sel_scores(sel_scores_row: np.ndarray, idx_row: np.ndarray, ref_scores: np.ndarray,
                     c: int, k: int):
    n = min(k, c + 1)
    sel = np.asarray(idx_row)[: n - 1]
    got = np.asarray(sel_scores_row, dtype=np.float64)
    assert got[n - 1] == np.inf, "own block score must be +inf"
    assert np.all(np.isneginf(got[n:])), "padding scores must be -inf"
    if n > 1:
        tau = score_tau(ref_scores[:c])
        err = np.abs(got[: n - 1] - ref_scores[sel])
        assert err.max() <= tau, f"score error {err.max():.3g} > tau {tau:.3g}"
        return float(err.max() / max(tau, 1e-300) * SCORE_RTOL)
    return 0.0


def check_attention(out_gpu_bits: np.ndarray, out_ref: np.ndarray, lse_gpu=None, lse_ref=None
                    ) -> dict:
    g = widen(out_gpu_bits).reshape(out_ref.shape)
    err = np.abs(g - out_ref)
    tol = ATTN_MAX_ABS + np.where(np.abs(out_ref) >= 4.0, 0.5 * ulp_bf16(out_ref), 0.0)
    worst = float(err.max())
    assert np.all(err <= tol), f"attention max-abs error {worst:.4g} > {ATTN_MAX_ABS}"
    rel = float(np.linalg.norm(g - out_ref) / max(np.linalg.norm(out_ref), 1e-300))
    assert rel <= ATTN_REL_L2, f"attention rel-L2 {rel:.4g} > {ATTN_REL_L2}"
    res = {"attn_max_abs": worst, "attn_rel_l2": rel}
    if lse_gpu is not None:
        le = float(np.max(np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)))
        assert le <= LSE_ABS, f"lse error {le:.4g} > {LSE_ABS}"
        res["lse_max_abs"] = le
    return res


# Gradients of the fixed-selection backward: the matrix-core products take bf16 operands
# (2^-9 relative each: the softmax weights, dz, q, dA), D = dout . out uses the bf16 forward
# output, and dz = P (dP - D) cancels where dP ~ D.  Bound: relative L2 within 5x the bf16
# step, and no element further than 3 % of the tensor's largest magnitude from the oracle.
GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 3e-2


def check_grad(name: str, gpu: np.ndarray, ref: np.ndarray) -> dict:
    g = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
    err = np.abs(g - ref)
    scale = max(float(np.abs(ref).max()), 1e-300)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float(err.max() / scale)
    assert rel <= GRAD_REL_L2, f"{name}: relative L2 error {rel:.4g} > {GRAD_REL_L2}"
    assert worst <= GRAD_MAX_REL, f"{name}: max error {worst:.4g} of max|ref| > {GRAD_MAX_REL}"
    return {f"{name}_rel_l2": rel, f"{name}_max_rel": worst}


def stratified_rows(q_start: int, T: int, B: int, k: int, n_random: int, seed: int,
                    extra=()) -> np.ndarray:
    """Query rows to check at full size: block edges, the k*B regime edge, chunk edges,
    the last row, and seeded random rows (row indices relative to q_start)."""
    cand = {0, 1, T - 1, T - 2}
    for t in (0, 1, B - 1, B, 2 * B - 1, k * B - 1, k * B, k * B + 1, (k - 1) * B, (k + 1) * B - 1):
        cand.add(t - q_start)
    pos_last = q_start + T - 1
    cand.add(pos_last - q_start - (pos_last % B))  # first token of the last block
    for e in extra:
        cand.add(int(e))
    rng = np.random.default_rng(seed)
    cand.update(rng.integers(0, T, size=n_random).tolist())
    rows = np.array(sorted(r for r in cand if 0 <= r < T), dtype=np.int64)
    return rows
