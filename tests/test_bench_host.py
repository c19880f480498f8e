"""Host-side logic of the benchmark (CPU): its refusal of more than one GPU, and the work
counts its rooflines divide by, checked against the oracle's own selection on small cases.

The attention's algorithmic flop count is 4 d Hq per attended (query, token) pair and the
indexer's is 2 P per scored (query, block) pair; bench.attended_pairs and bench.scored_pairs
count those pairs from the selection rule in closed form.  Here the same counts come from the
oracle: the token sets of its causal top-k (ai.info "Sparse GQA targets million-token context":
top-k blocks of eight tokens; the own block kept) and the candidates its scores cover.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("B,k,q_start,T", [(8, 16, 0, 700), (8, 16, 517, 300), (1, 5, 0, 64),
                                           (4, 3, 9, 97), (16, 4, 0, 300)])
def test_attended_and_scored_pairs_match_the_oracle(B, k, q_start, T):
    rng = np.random.default_rng(B * 1000 + k + q_start)
    t = np.arange(q_start, q_start + T, dtype=np.int64)
    width = max(1, int(t.max()) // B)
    # random scores over every candidate column; the oracle masks what a row may not score
    P = 8
    qp = rng.standard_normal((T, P)).astype(np.float32)
    qp_bits = (qp.view(np.uint32) >> 16).astype(np.uint16)
    kb = rng.standard_normal((width + 1, P))
    sc = oracle.scores(qp_bits, t, B, kb, width=width)
    # scored pairs: the finite entries of each row (complete past blocks only)
    assert int(np.isfinite(sc).sum()) == bench.scored_pairs(q_start, T, B)
    idx = oracle.topk(sc, t, B, k)
    attended = sum(len(oracle.token_set(idx[i], B, int(t[i]))) for i in range(T))
    assert attended == bench.attended_pairs(q_start, T, B, k)
