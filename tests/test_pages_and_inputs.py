"""Pins from the pages' printed figures, and statistics of the synthetic input recipe (CPU)."""
import json
import math
import os

import numpy as np
import torch

import oracle
from long_context_sparse_18_amd import REAL, WORKLOADS
from long_context_sparse_18_amd import inputs
from long_context_sparse_18_amd.configs import Workload, LayerShape

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def g(name):
    return GOLD[name]["value"]


def test_real_shape_matches_pages():
    assert REAL.num_q_heads == g("num_attention_heads")
    assert REAL.num_kv_heads == g("num_attention_groups")
    assert REAL.head_dim == g("head_dim")
    assert REAL.proxy_dim == g("proxy_dim")
    assert REAL.block_size == g("block_size")
    assert REAL.topk_blocks == g("sparse_topk_blocks")
    # "top-k 4096" with blocks of 8 is the catalogue's topk 512 counted in blocks
    assert REAL.topk_blocks * REAL.block_size == g("topk_tokens")


def test_kv_bytes_per_token():
    per_layer = 2 * REAL.num_kv_heads * REAL.head_dim * 2  # K and V, bf16
    assert per_layer * g("full_attention_layers") == g("kv_bytes_per_token_full_layers")
    assert per_layer * g("backbone_layers") == g("kv_bytes_per_token_if_all_global")
    # the decode workload's cache: one layer, one 1M-token sequence = 3 GiB
    assert per_layer * WORKLOADS[3].L == 3 * 2**30
    assert WORKLOADS[3].L == g("max_position_embeddings")


def test_indexer_work_cut_is_eight():
    """Scored (query, candidate) pairs at B=8 vs B=1: sum floor(t/8) / sum t = (T/8-1)/(T-1),
    which tends to the pages' 8x cut."""
    for T in (1024, 32768, 131072):
        t = np.arange(T)
        pairs8 = int(np.sum(t // 8))
        pairs1 = int(np.sum(t // 1))
        assert pairs8 / pairs1 == (T / 8 - 1) / (T - 1)
        assert abs(pairs1 / pairs8 - g("indexer_cost_cut")) < 8 * 8.0 / T + 1e-9
    # and the oracle counts candidates the same way
    for t in (0, 7, 8, 9, 1048575):
        assert oracle.num_candidates(t, 8) == t // 8
        assert oracle.num_candidates(t, 1) == t
    # the index itself has 1/8 the rows
    assert oracle.num_blocks(131072, 8) * 8 == oracle.num_blocks(131072, 1)


def test_chunked_prefill_workload_arithmetic():
    wl = WORKLOADS[4]
    assert wl.q_start + wl.T == wl.L == 1048580
    assert wl.q_start // 8 == 130048 and wl.q_start % 8 == 4
    assert wl.nblk == 131073           # last block holds 4 tokens
    assert (wl.L - 1) // 8 == 131072   # the last query scores 131 072 candidate blocks


def _small(rho=0.9, reseed=None, L=8192):
    return Workload("stat", LayerShape(8, 2, 64, 32, 8, 16), 1, 16, L, L - 16, reseed, rho)


def test_ar1_key_statistics():
    wl = _small()
    x = inputs.ar1_stream(wl.L, 128, inputs._gen(0, "K", 0, "cpu"), "cpu", 0.9).double().numpy()
    var = x.var()
    lag1 = np.mean(x[1:] * x[:-1]) / var
    assert abs(var - 1.0) < 0.05, var
    assert abs(lag1 - 0.9) < 0.01, lag1
    # block means of 8: variance (1/64) sum_{a,b} 0.9^|a-b| = 0.7732
    want = sum(0.9 ** abs(a - b) for a in range(8) for b in range(8)) / 64
    bm = x[: wl.L // 8 * 8].reshape(-1, 8, 128).mean(axis=1)
    assert abs(want - 0.7732) < 1e-4
    assert abs(bm.var() - want) < 0.04, bm.var()


def test_ar1_restart_decorrelates():
    x = inputs.ar1_stream(4096, 512, inputs._gen(0, "K", 0, "cpu"), "cpu", 0.9,
                          reseed_every=1024).double().numpy()
    across = [np.corrcoef(x[b - 1], x[b])[0, 1] for b in (1024, 2048, 3072)]
    within = [np.corrcoef(x[b], x[b + 1])[0, 1] for b in (1024, 2048, 3072)]
    assert all(abs(c) < 0.15 for c in across), across
    assert all(c > 0.8 for c in within), within


def test_generator_is_seeded_and_shaped():
    wl = WORKLOADS[0]
    a = inputs.make_prefill(wl, 0, "cpu")
    b = inputs.make_prefill(wl, 0, "cpu")
    c = inputs.make_prefill(wl, 1, "cpu")
    for key in a:
        assert torch.equal(a[key], b[key]), key
        assert not torch.equal(a[key], c[key]), key
        assert a[key].dtype == torch.bfloat16
    s = wl.shape
    assert a["Q"].shape == (wl.T, s.num_q_heads, s.head_dim)
    assert a["K"].shape == (wl.L, s.num_kv_heads, s.head_dim)
    assert a["kp"].shape == (wl.L, s.proxy_dim) and a["qp"].shape == (wl.T, s.proxy_dim)
    assert a["G"].shape == (wl.T, s.num_q_heads)
    # proxies have O(1) spread (weights scaled by 1/sqrt(fan_in))
    assert 0.5 < a["kp"].float().std().item() < 1.5
    assert 0.05 < a["qp"].float().std().item() < 1.0
