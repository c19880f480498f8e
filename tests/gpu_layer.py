"""Run the HIP path through the C ABI and check it against the oracle (GPU tests only)."""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
from long_context_sparse_18_amd import sgqa
from long_context_sparse_18_amd.inputs import bits
import parity


def say(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def run_prefill(shape, d, q_start: int, L: int, workspace=None, kb=None, build_index=True,
                attn_workspace=None):
    """index_build -> indexer_topk -> sparse_attn_prefill for one sequence."""
    dev = d["Q"].device
    T = d["Q"].shape[0]
    B, k, P = shape.block_size, shape.topk_blocks, shape.proxy_dim
    nblk = -(-L // B)
    if kb is None:
        kb = torch.empty((nblk, P), dtype=torch.bfloat16, device=dev)
    if build_index:
        sgqa.index_build(shape, d["kp"], kb, [L])
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    sel = torch.empty((T, k), dtype=torch.float32, device=dev)
    sgqa.indexer_topk(shape, d["qp"], kb, [q_start], idx, sel, workspace=workspace)
    out = torch.empty_like(d["Q"])
    lse = torch.empty((T, shape.num_q_heads), dtype=torch.float32, device=dev)
    sgqa.sparse_attn_prefill(shape, d["Q"], d["K"], d["V"], d["G"], idx, q_start, L,
                             1.0 / math.sqrt(shape.head_dim), out, lse, workspace=attn_workspace)
    torch.cuda.synchronize()
    return dict(kb=kb, idx=idx, sel=sel, out=out, lse=lse)


def check_prefill_rows(shape, d, res, q_start: int, rows: np.ndarray, kb_ref=None,
                       host_cache=None) -> dict:
    """Stage-isolated and end-to-end checks of the given query rows (relative to q_start)."""
    B, k = shape.block_size, shape.topk_blocks
    rows = np.asarray(rows, dtype=np.int64)
    t = rows + q_start
    kb_gpu = parity.widen(bits(res["kb"]))
    if kb_ref is None:
        kb_ref = oracle.index_build(bits(d["kp"]), B)
    width = max(1, int(t.max()) // B)
    rows_t = torch.from_numpy(rows).to(res["idx"].device)
    qp_rows = bits(d["qp"].index_select(0, rows_t))
    idx_rows = res["idx"].index_select(0, rows_t).cpu().numpy()
    sel_rows = res["sel"].index_select(0, rows_t).cpu().numpy()
    # stage-isolated: scores from the GPU's own bf16 kb
    s_iso = oracle.scores(qp_rows, t, B, kb_gpu, width=width)
    ref_iso = oracle.topk(s_iso, t, B, k)
    # end-to-end: scores from the oracle's fp64 kb
    s_e2e = oracle.scores(qp_rows, t, B, kb_ref, width=width)
    ref_e2e = oracle.topk(s_e2e, t, B, k)
    exact_iso = exact_e2e = 0
    worst_score = 0.0
    for r in range(len(rows)):
        c = int(t[r] // B)
        exact_iso += parity.check_selection(idx_rows[r], s_iso[r], c, k, ref_iso[r])
        exact_e2e += parity.check_selection(idx_rows[r], s_e2e[r], c, k, ref_e2e[r],
                                            end_to_end=True)
        worst_score = max(worst_score, parity.check_sel_scores(sel_rows[r], idx_rows[r], s_iso[r], c, k))
    # attention given the GPU's selection
    if host_cache is None:
        host_cache = (bits(d["K"]), bits(d["V"]))
    q_rows = bits(d["Q"].index_select(0, rows_t))
    g_rows = bits(d["G"].index_select(0, rows_t))
    out_ref, lse_ref = oracle.sparse_attention(q_rows, t, host_cache[0], host_cache[1], g_rows,
                                               idx_rows, B, 1.0 / math.sqrt(shape.head_dim))
    att = parity.check_attention(bits(res["out"].index_select(0, rows_t)), out_ref,
                                 res["lse"].index_select(0, rows_t).cpu().numpy(), lse_ref)
    return dict(rows=len(rows), exact_iso=exact_iso, exact_e2e=exact_e2e,
                worst_score_rel=worst_score, **att)
