"""GPU parity on the tiny layer (8 query heads, 2 KV heads, d 64, proxy 32): every row,
every stage, plus the edge cases (k = all, k = 1, B = 1, mid-block chunks, several
sequences, decode with mixed cache lengths, small workspaces, empty calls)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from gpu_layer import check_prefill_rows, run_prefill, say
from long_context_sparse_18_amd import WORKLOADS, inputs, probe, sgqa
from long_context_sparse_18_amd.configs import Workload, with_selection
from long_context_sparse_18_amd.inputs import bits

pytestmark = pytest.mark.gpu

WL = WORKLOADS[0]
DEV = "cuda"


@pytest.fixture(scope="module")
def tiny():
    say("tiny: generating inputs")
    return inputs.make_prefill(WL, 0, DEV)


@pytest.fixture(scope="module")
def tiny_host(tiny):
    return bits(tiny["K"]), bits(tiny["V"])


def test_tiny_index_build(tiny):
    say("tiny: index_build")
    kb = torch.empty((WL.nblk, WL.shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(WL.shape, tiny["kp"], kb, [WL.L])
    torch.cuda.synchronize()
    st = parity.check_kb(bits(kb), oracle.index_build(bits(tiny["kp"]), 8))
    assert st["kb_bit_equal_to_rne"] >= 0.999, st


@pytest.mark.parametrize("B,k", [(8, 16), (8, 128), (8, 1), (1, 16), (1, 1024), (8, 3)])
def test_tiny_full_layer_every_row(tiny, tiny_host, B, k):
    shape = with_selection(WL.shape, B, k)
    say(f"tiny: layer B={B} k={k}")
    res = run_prefill(shape, tiny, 0, WL.L)
    rows = np.arange(WL.T)
    st = check_prefill_rows(shape, tiny, res, 0, rows, host_cache=tiny_host)
    say(f"tiny B={B} k={k}: {st}")
    assert st["exact_iso"] >= len(rows) - 2


def test_tiny_dense_selection_matches_sdpa(tiny):
    """k covers every block: the layer is dense causal gated GQA (torch SDPA in fp32 on the
    CPU as a second, independent reference next to the oracle)."""
    shape = with_selection(WL.shape, 8, 128)
    res = run_prefill(shape, tiny, 0, WL.L)
    Q = tiny["Q"].float().cpu().permute(1, 0, 2)
    K = tiny["K"].float().cpu().permute(1, 0, 2).repeat_interleave(4, dim=0).contiguous()
    V = tiny["V"].float().cpu().permute(1, 0, 2).repeat_interleave(4, dim=0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    o = o.permute(1, 0, 2) * torch.sigmoid(tiny["G"].float().cpu())[:, :, None]
    got = res["out"].float().cpu()
    assert (got - o).abs().max().item() < 1e-2
    assert ((got - o).norm() / o.norm()).item() < 5e-3


@pytest.mark.parametrize("rows_per_chunk", [1000, 300, 1])
def test_tiny_sliced_prefill_matches(tiny, tiny_host, rows_per_chunk):
    """With a workspace the selected blocks are visited in history slices, with the softmax
    state carried between launches, in row chunks that fit the workspace: same result as the
    single pass up to fp32 summation order, and oracle parity on every row."""
    shape = WL.shape
    per_row = sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, shape, 1, 1, WL.L)
    ws = torch.empty(per_row * rows_per_chunk, dtype=torch.uint8, device=DEV)
    one = run_prefill(shape, tiny, 0, WL.L)
    sliced = run_prefill(shape, tiny, 0, WL.L, attn_workspace=ws)
    assert torch.equal(one["idx"], sliced["idx"])
    diff = (one["out"].float() - sliced["out"].float()).abs().max().item()
    assert diff <= 2 ** -6, diff
    st = check_prefill_rows(shape, tiny, sliced, 0, np.arange(WL.T), host_cache=tiny_host)
    say(f"tiny sliced ({rows_per_chunk} rows/chunk): {st}")


@pytest.mark.parametrize("chunks", [1, 3, 8])
def test_tiny_layer_schedule_same_bits(tiny, chunks):
    """The layer schedule in row chunks (each chunk's selection, then its attention) gives the
    bits of the stages run one after the other over all rows (uneven chunks)."""
    from long_context_sparse_18_amd import layer
    shape = WL.shape
    ws_a = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, shape, 1, WL.T, WL.L),
                       dtype=torch.uint8, device=DEV)
    ref = run_prefill(shape, tiny, 0, WL.L, attn_workspace=ws_a)
    kb = torch.empty_like(ref["kb"])
    idx = torch.full_like(ref["idx"], -7)
    out = torch.empty_like(ref["out"])
    lse = torch.empty_like(ref["lse"])
    ws_t = torch.empty(sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, shape, 1, WL.T, WL.L),
                       dtype=torch.uint8, device=DEV)
    layer.prefill_layer(shape, tiny, 0, WL.L, 1.0 / math.sqrt(shape.head_dim), kb, idx, out,
                        lse, ws_t, ws_a, chunks=chunks)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref["idx"]) and torch.equal(out, ref["out"])
    assert torch.equal(lse, ref["lse"]) and torch.equal(kb, ref["kb"])


def test_prefill_resident_and_long_rows_in_one_call():
    """With a workspace, rows whose histories span at most 16 ranges of 5k blocks (here
    16 x 80 blocks = 10240 tokens) take the resident prefill and the longer ones the sliced
    launches (one pass each).  A call over 12288 rows uses both; calls over row chunks that cut
    across that boundary and elsewhere give the same bits, and rows on both sides of it match
    the oracle."""
    shape = WL.shape
    wl = Workload("tiny-12k", shape, nseq=1, T=12288, L=12288, q_start=0)
    say("resident + long rows: generating")
    d = inputs.make_prefill(wl, 11, DEV)
    ws = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, shape, 1, wl.T, wl.L),
                     dtype=torch.uint8, device=DEV)
    res = run_prefill(shape, d, 0, wl.L, attn_workspace=ws)
    out = torch.full_like(res["out"], 7.0)
    lse = torch.full_like(res["lse"], 7.0)
    scale = 1.0 / math.sqrt(shape.head_dim)
    bounds = [0, 3001, 10239, 10241, 12288]
    for r0, r1 in zip(bounds[:-1], bounds[1:]):
        sgqa.sparse_attn_prefill(shape, d["Q"][r0:r1], d["K"], d["V"], d["G"][r0:r1],
                                 res["idx"][r0:r1], r0, wl.L, scale, out[r0:r1], lse[r0:r1],
                                 workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, res["out"]) and torch.equal(lse, res["lse"])
    rows = np.array([0, 7, 1000, 5000, 10230, 10238, 10239, 10240, 10241, 10250, 12000, 12287])
    st = check_prefill_rows(shape, d, res, 0, rows)
    say(f"resident + long rows: {st}")
    assert st["exact_iso"] >= len(rows) - 1


def test_tiny_deterministic(tiny):
    a = run_prefill(WL.shape, tiny, 0, WL.L)
    b = run_prefill(WL.shape, tiny, 0, WL.L)
    for key in ("kb", "idx", "sel", "out", "lse"):
        assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), key


def test_tiny_small_workspace_same_selection(tiny):
    """A workspace that holds only 64 query rows forces 16 passes; the result is identical."""
    full = run_prefill(WL.shape, tiny, 0, WL.L)
    ld = 128  # round_up(127, 64)
    ws = torch.empty(64 * ld * 4, dtype=torch.uint8, device=DEV)
    small = run_prefill(WL.shape, tiny, 0, WL.L, workspace=ws)
    assert torch.equal(full["idx"], small["idx"])
    assert torch.equal(full["out"], small["out"])


def test_tiny_chunk_starting_mid_block(tiny, tiny_host):
    """Queries [517, 817) on a cache of 817 tokens; the index range the chunk touched is
    rebuilt after the rest of the index was built; the trailing block holds 1 token."""
    q0, L = 517, 817
    d = {k_: v[:L] for k_, v in tiny.items() if k_ in ("K", "V", "kp")}
    d.update({k_: tiny[k_][q0:L] for k_ in ("Q", "G", "qp")})
    shape = WL.shape
    nblk = -(-L // 8)
    kb = torch.zeros((nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, d["kp"], kb, [L], 0, q0 // 8)       # history blocks
    sgqa.index_build(shape, d["kp"], kb, [L], q0 // 8, -1)      # blocks the chunk touched
    res = run_prefill(shape, d, q0, L, kb=kb, build_index=False)
    parity.check_kb(bits(kb), oracle.index_build(bits(d["kp"]), 8))
    st = check_prefill_rows(shape, d, res, q0, np.arange(L - q0),
                            host_cache=(tiny_host[0][:L], tiny_host[1][:L]))
    say(f"tiny chunk: {st}")


def test_tiny_several_sequences_topk(tiny):
    """Three sequences with different query starts in one indexer call."""
    shape = WL.shape
    T = 200
    starts = [0, 333, 824]
    kb = torch.empty((WL.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, tiny["kp"], kb, [WL.L])
    qp = torch.stack([tiny["qp"][s:s + T] for s in starts])
    kb3 = kb.unsqueeze(0).expand(3, -1, -1).contiguous()
    idx = torch.empty((3, T, shape.topk_blocks), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb3, starts, idx)
    torch.cuda.synchronize()
    kb_gpu = parity.widen(bits(kb))
    for si, s in enumerate(starts):
        t = np.arange(s, s + T)
        sc = oracle.scores(bits(qp[si]), t, 8, kb_gpu, width=WL.nblk)
        ref = oracle.topk(sc, t, 8, shape.topk_blocks)
        got = idx[si].cpu().numpy()
        for r in range(T):
            parity.check_selection(got[r], sc[r], int(t[r] // 8), shape.topk_blocks, ref[r])


def test_tiny_decode_mixed_lengths(tiny):
    """Decode for 5 sequences whose caches hold 1, 9, 130, 1000 and 1024 tokens."""
    shape = WL.shape
    lens = [1, 9, 130, 1000, 1024]
    n = len(lens)
    Lmax = WL.L
    K = tiny["K"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    V = tiny["V"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    kp = tiny["kp"].unsqueeze(0).expand(n, -1, -1).contiguous()
    Q = torch.stack([tiny["Q"][L_ - 1] for L_ in lens])
    G = torch.stack([tiny["G"][L_ - 1] for L_ in lens])
    qp = torch.stack([tiny["qp"][L_ - 1] for L_ in lens]).unsqueeze(1)
    kb = torch.empty((n, WL.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, kp, kb, lens)
    idx = torch.empty((n, 1, shape.topk_blocks), dtype=torch.int32, device=DEV)
    sel = torch.empty((n, 1, shape.topk_blocks), dtype=torch.float32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1 for L_ in lens], idx, sel)
    out = torch.empty_like(Q)
    lse = torch.empty((n, shape.num_q_heads), dtype=torch.float32, device=DEV)
    sgqa.sparse_attn_decode(shape, Q, K, V, G, idx.view(n, -1), lens,
                            1.0 / math.sqrt(shape.head_dim), out, lse)
    torch.cuda.synchronize()
    Kb, Vb = bits(tiny["K"]), bits(tiny["V"])
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        kb_ref = oracle.index_build(bits(tiny["kp"][:L_]), 8)
        nb = -(-L_ // 8)
        parity.check_kb(bits(kb[b, :nb]), kb_ref)
        sc = oracle.scores(bits(qp[b]), t, 8, parity.widen(bits(kb[b, :nb])), width=max(1, nb))
        ref = oracle.topk(sc, t, 8, shape.topk_blocks)
        got = idx[b, 0].cpu().numpy()
        parity.check_selection(got, sc[0], int(t[0] // 8), shape.topk_blocks, ref[0])
        o_ref, l_ref = oracle.sparse_attention(bits(Q[b:b + 1]), t, Kb[:L_], Vb[:L_],
                                               bits(G[b:b + 1]), got[None, :], 8,
                                               1.0 / math.sqrt(shape.head_dim))
        parity.check_attention(bits(out[b:b + 1]), o_ref, lse[b:b + 1].cpu().numpy(), l_ref)


def test_tiny_empty_calls_are_noops(tiny):
    shape = WL.shape
    out = torch.full((1, shape.num_q_heads, shape.head_dim), 7.0, dtype=torch.bfloat16, device=DEV)
    sgqa.sparse_attn_prefill(shape, tiny["Q"][:0], tiny["K"], tiny["V"], tiny["G"][:0],
                             torch.empty((0, shape.topk_blocks), dtype=torch.int32, device=DEV),
                             0, WL.L, 0.125, out)
    idx = torch.full((1, shape.topk_blocks), 5, dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, tiny["qp"][:0], tiny["kp"][:16], [0], idx)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(idx == 5)


@pytest.mark.parametrize("k", [16, 300])
def test_decode_topk_many_chunks(k):
    """One query per sequence against long indexes (up to 25 000 blocks), so the decode
    top-k splits the candidates over several chunks; checked against the oracle."""
    lens = [70001, 131072, 200003, 9]
    Lmax = max(lens)
    shape = with_selection(WL.shape, 8, k)
    wl = Workload("tiny-long", shape, nseq=len(lens), T=1, L=Lmax, q_start=Lmax - 1)
    n = len(lens)
    kp = torch.empty((n, Lmax, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    qp = torch.empty((n, 1, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    for b in range(n):
        _, _, kpb = inputs.make_cache(wl, 7, DEV, seq=b)
        kp[b].copy_(kpb)
        qp[b, 0].copy_(inputs.make_queries(wl, 7, DEV, seq=b, T=1)[2][0])
    nblk = -(-Lmax // 8)
    kb = torch.empty((n, nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, kp, kb, lens)
    idx = torch.empty((n, 1, k), dtype=torch.int32, device=DEV)
    sel = torch.empty((n, 1, k), dtype=torch.float32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1 for L_ in lens], idx, sel)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        c = int(t[0] // 8)
        kbw = parity.widen(bits(kb[b, : -(-L_ // 8)]))
        sc = oracle.scores(bits(qp[b]), t, 8, kbw, width=max(1, c))
        ref = oracle.topk(sc, t, 8, k)
        got = idx[b, 0].cpu().numpy()
        assert parity.check_selection(got, sc[0], c, k, ref[0]) or c > 1000
        parity.check_sel_scores(sel[b, 0].cpu().numpy(), got, sc[0], c, k)


@pytest.mark.parametrize("window", [1, 8, 17, 512, 5000])
def test_tiny_sliding_window_every_row(tiny, tiny_host, window):
    """Gated sliding-window attention on every row of the tiny layer, against the oracle."""
    shape = WL.shape
    out = torch.empty_like(tiny["Q"])
    lse = torch.empty((WL.T, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.swa_prefill(shape, tiny["Q"], tiny["K"], tiny["V"], tiny["G"], 0, WL.L, window, scale,
                     out, lse)
    torch.cuda.synchronize()
    t = np.arange(WL.T)
    o_ref, l_ref = oracle.window_attention(bits(tiny["Q"]), t, tiny_host[0], tiny_host[1],
                                           bits(tiny["G"]), window, scale)
    parity.check_attention(bits(out), o_ref, lse.cpu().numpy(), l_ref)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.4])
def test_tiny_sliding_window_scales(tiny, tiny_host, scale):
    """The sliding-window kernel applies the scale inside the exponent, after the maximum:
    a negative scale (scores negated first), a zero scale (equal weights over the window)
    and a large one, on every row against the oracle, at window 17 and 300."""
    shape = WL.shape
    t = np.arange(WL.T)
    for window in (17, 300):
        out = torch.empty_like(tiny["Q"])
        lse = torch.empty((WL.T, shape.num_q_heads), dtype=torch.float32, device=DEV)
        sgqa.swa_prefill(shape, tiny["Q"], tiny["K"], tiny["V"], tiny["G"], 0, WL.L, window,
                         scale, out, lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.window_attention(bits(tiny["Q"]), t, tiny_host[0], tiny_host[1],
                                               bits(tiny["G"]), window, scale)
        parity.check_attention(bits(out), o_ref, lse.cpu().numpy(), l_ref)


def test_tiny_sliding_window_peaked(tiny, tiny_host):
    """A scale of 30: each query's softmax is close to one-hot and its logits span several
    hundred log2 units, so a running maximum taken over only some of a query's scores (a wrong
    lane exchange in the cross-row maximum) would overflow the weights to inf.  Output to the
    usual bounds; lse (up to ~1400) to 2e-2 plus 1e-5 of its size: the fp32 dot products of 64
    terms carry up to ~2e-4 of rounding, times the scale of 30."""
    shape = WL.shape
    t = np.arange(WL.T)
    for window in (17, 300):
        out = torch.empty_like(tiny["Q"])
        lse = torch.empty((WL.T, shape.num_q_heads), dtype=torch.float32, device=DEV)
        sgqa.swa_prefill(shape, tiny["Q"], tiny["K"], tiny["V"], tiny["G"], 0, WL.L, window,
                         30.0, out, lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.window_attention(bits(tiny["Q"]), t, tiny_host[0], tiny_host[1],
                                               bits(tiny["G"]), window, 30.0)
        assert np.abs(l_ref).max() > 100.0  # the logits really are spread wide
        parity.check_attention(bits(out), o_ref)
        got = lse.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - l_ref) <= 2e-2 + 1e-5 * np.abs(l_ref))


def test_tiny_sliding_window_chunk_mid_sequence(tiny, tiny_host):
    """Queries [300, 700) of a 700-token cache with a window of 64."""
    shape = WL.shape
    q0, L, W = 300, 700, 64
    out = torch.empty_like(tiny["Q"][q0:L])
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.swa_prefill(shape, tiny["Q"][q0:L], tiny["K"][:L], tiny["V"][:L], tiny["G"][q0:L], q0, L,
                     W, scale, out)
    torch.cuda.synchronize()
    t = np.arange(q0, L)
    o_ref, _ = oracle.window_attention(bits(tiny["Q"][q0:L]), t, tiny_host[0][:L],
                                       tiny_host[1][:L], bits(tiny["G"][q0:L]), W, scale)
    parity.check_attention(bits(out), o_ref)


def _integer_index(shape, n, nblk, seed):
    """kb and qp with small integer entries: every score is an exact integer in fp32 and
    fp64 alike, so heavy exact ties are common and the selection is fully determined by
    the lowest-index rule."""
    g = torch.Generator().manual_seed(seed)
    kb = torch.randint(-2, 3, (n, nblk, shape.proxy_dim), generator=g).to(torch.bfloat16)
    return kb


@pytest.mark.parametrize("k", [16, 512, 3000])
def test_decode_topk_exact_ties(k):
    """Decode top-k on integer-valued scores (many exact ties, one all-zero query so that
    every score ties): the selection and its scores must equal the oracle's exactly."""
    lens = [1048576, 400003, 9, 5000]
    n, Lmax = len(lens), max(lens)
    shape = with_selection(WL.shape, 8, k)
    nblk = -(-Lmax // 8)
    kb = _integer_index(shape, n, nblk, 11 + k).to(DEV)
    g = torch.Generator().manual_seed(5)
    qp = torch.randint(-2, 3, (n, 1, shape.proxy_dim), generator=g).to(torch.bfloat16)
    qp[3].zero_()
    qp = qp.to(DEV)
    idx = torch.empty((n, 1, k), dtype=torch.int32, device=DEV)
    sel = torch.empty((n, 1, k), dtype=torch.float32, device=DEV)
    say(f"decode ties k={k}")
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1 for L_ in lens], idx, sel)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        c = int(t[0] // 8)
        kbw = parity.widen(bits(kb[b, : -(-L_ // 8)]))
        sc = oracle.scores(bits(qp[b]), t, 8, kbw, width=max(1, c))
        ref = oracle.topk(sc, t, 8, k)[0]
        got = idx[b, 0].cpu().numpy()
        assert np.array_equal(got, ref), f"seq {b}: selection differs"
        want = np.where(ref < 0, -np.inf, np.where(ref == c, np.inf, sc[0][np.clip(ref, 0, max(0, c - 1))]))
        assert np.array_equal(sel[b, 0].cpu().numpy().astype(np.float64), want)


def test_decode_topk_crowded_units():
    """Decode top-k where the blocks above the threshold crowd into the 16-block units that one
    wave of the select holds (units b * 1024 + lane, b < 8): 300 of them carry the top scores,
    more than the wave's share of the unit list, so the select takes its exact path over every
    key.  One sequence of 1 048 576 tokens, scores q . kb = kb[:, 0] exactly (one nonzero
    proxy dim); selection and scores must equal the oracle's exactly."""
    k, L_ = 512, 1048576
    shape = with_selection(WL.shape, 8, k)
    nblk = L_ // 8
    g = torch.Generator().manual_seed(21)
    kb = torch.zeros((1, nblk, shape.proxy_dim), dtype=torch.float32)
    kb[0, :, 0] = torch.randn(nblk, generator=g)
    units = [b * 1024 + lane for b in range(5) for lane in range(60)]
    for m, u in enumerate(units):
        kb[0, 16 * u + 5, 0] = 32.0 + (m % 64) / 4.0
    kb = kb.to(torch.bfloat16).to(DEV)
    qp = torch.zeros((1, 1, shape.proxy_dim), dtype=torch.bfloat16)
    qp[0, 0, 0] = 1.0
    qp = qp.to(DEV)
    idx = torch.empty((1, 1, k), dtype=torch.int32, device=DEV)
    sel = torch.empty((1, 1, k), dtype=torch.float32, device=DEV)
    say("decode crowded units")
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1], idx, sel)
    torch.cuda.synchronize()
    t = np.array([L_ - 1])
    c = int(t[0] // 8)
    kbw = parity.widen(bits(kb[0]))
    sc = oracle.scores(bits(qp[0]), t, 8, kbw, width=c)
    ref = oracle.topk(sc, t, 8, k)[0]
    got = idx[0, 0].cpu().numpy()
    assert np.array_equal(got, ref), "selection differs"
    assert set(16 * u + 5 for u in units) <= set(ref.tolist())
    want = np.where(ref == c, np.inf, sc[0][np.clip(ref, 0, c - 1)])
    assert np.array_equal(sel[0, 0].cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("q0", [30000, 8000])
def test_prefill_topk_exact_ties(q0):
    """Prefill top-k (one workgroup per query row) on integer-valued scores: exact.  Row 7 has
    all scores equal: with ~3 750 candidate blocks (q0 = 30000) more keys tie than the
    selection lists, so it takes the full-row path; with ~1 000 (q0 = 8000) the ties of the
    full key are broken inside the listed keys (lowest blocks first)."""
    k, T = 512, 96
    shape = with_selection(WL.shape, 8, k)
    nblk = -(-(q0 + T) // 8)
    kb = _integer_index(shape, 1, nblk, 3)[0].to(DEV)
    g = torch.Generator().manual_seed(9)
    qp = torch.randint(-2, 3, (T, shape.proxy_dim), generator=g).to(torch.bfloat16)
    qp[7].zero_()
    qp = qp.to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [q0], idx)
    torch.cuda.synchronize()
    t = np.arange(q0, q0 + T)
    sc = oracle.scores(bits(qp), t, 8, parity.widen(bits(kb)), width=int(t.max()) // 8)
    ref = oracle.topk(sc, t, 8, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.gpu
def test_prefill_topk_every_row_falls_back():
    """Every row's list overflows (all scores tie: zero query proxies), so all 300 rows are
    queued and the 64 persistent fallback workgroups each take several of them: the result is
    the lowest k-1 blocks plus the own block, with their scores, as the oracle has it."""
    k, T, q0 = 512, 300, 30000
    shape = with_selection(WL.shape, 8, k)
    nblk = -(-(q0 + T) // 8)
    kb = _integer_index(shape, 1, nblk, 5)[0].to(DEV)
    qp = torch.zeros((T, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    sel = torch.empty((T, k), dtype=torch.float32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [q0], idx, sel)
    torch.cuda.synchronize()
    t = np.arange(q0, q0 + T)
    sc = oracle.scores(bits(qp), t, 8, parity.widen(bits(kb)), width=int(t.max()) // 8)
    ref = oracle.topk(sc, t, 8, k)
    assert np.array_equal(idx.cpu().numpy(), ref)
    got = sel.cpu().numpy()
    assert np.all(got[:, : k - 1] == 0.0) and np.all(np.isinf(got[:, k - 1]))


def test_prefill_topk_several_passes_same_bits(tiny):
    """A workspace that holds exactly one 64-row pass of the selection without a score matrix
    (the layer's 1024 rows in 16 passes) gives the bits of the one-pass call, scores included."""
    shape = with_selection(WL.shape, 8, 16)
    kb = torch.empty((WL.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, tiny["kp"], kb, [WL.L])
    full_idx = torch.empty((WL.T, 16), dtype=torch.int32, device=DEV)
    full_sel = torch.empty((WL.T, 16), dtype=torch.float32, device=DEV)
    sgqa.indexer_topk(shape, tiny["qp"], kb, [0], full_idx, full_sel)
    # fixed part: 256 B of counters + 64 fallback rows of ld = 128 floats; per row: 1024
    # sample keys, threshold, count, queue slot, 2048 listed (key, block) pairs
    ws = torch.empty(256 + 64 * 128 * 4 + 64 * (1024 * 4 + 12 + 2048 * 8), dtype=torch.uint8,
                     device=DEV)
    idx = torch.full_like(full_idx, -7)
    sel = torch.empty_like(full_sel)
    sgqa.indexer_topk(shape, tiny["qp"], kb, [0], idx, sel, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, full_idx)
    assert torch.equal(sel.view(torch.int32), full_sel.view(torch.int32))


def test_prefill_topk_sample_bound_too_high():
    """Prefill top-k when the sampled lower bound of the threshold overshoots: only every 16th
    block scores above -1 (exactly the blocks a 1024-key sample of a ~16 000-block row reads,
    with integer values that tie), so fewer than k-1 blocks reach the sample's bound and the
    full-row selection must give the oracle's exact result, ties to the lowest block."""
    k, T, q0 = 512, 8, 128000
    shape = with_selection(WL.shape, 8, k)
    nblk = -(-(q0 + T) // 8)
    j = torch.arange(nblk)
    kb = torch.zeros((nblk, shape.proxy_dim))
    kb[:, 0] = torch.where(j % 16 == 0, (j // 16) % 256, torch.full_like(j, -1)).float()
    kb = kb.to(torch.bfloat16).to(DEV)
    qp = torch.zeros((T, shape.proxy_dim))
    qp[:, 0] = 1.0
    qp = qp.to(torch.bfloat16).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [q0], idx)
    torch.cuda.synchronize()
    t = np.arange(q0, q0 + T)
    sc = oracle.scores(bits(qp), t, 8, parity.widen(bits(kb)), width=int(t.max()) // 8)
    ref = oracle.topk(sc, t, 8, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def _w_kt(wl, seed):
    """The key projection of the synthetic recipe as bf16 W^T [P, Hkv*d]."""
    return inputs.proxy_weights(wl, seed, DEV)[1].t().contiguous().to(torch.bfloat16)


@pytest.mark.parametrize("B", [8, 1, 32])
def test_tiny_index_from_keys(tiny, B):
    """Fused index maintenance on three sequences of different lengths (full and partial
    trailing blocks) against the oracle; then a one-block refresh leaves the rest untouched."""
    shape = with_selection(WL.shape, B, 16)
    lens = [1024, 1000, 37]
    n, Lmax = len(lens), max(lens)
    K = torch.zeros((n, Lmax) + tuple(tiny["K"].shape[1:]), dtype=torch.bfloat16, device=DEV)
    for b, L_ in enumerate(lens):
        K[b, :L_] = tiny["K"][:L_].roll(shifts=97 * b, dims=0)
    wkt = _w_kt(WL, 3)
    nblk = -(-Lmax // B)
    kb = torch.full((n, nblk, shape.proxy_dim), 7.0, dtype=torch.bfloat16, device=DEV)
    sgqa.index_build_from_keys(shape, K, wkt, kb, lens)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        ref = oracle.index_build_from_keys(bits(K[b, :L_]), bits(wkt), B)
        st = parity.check_kb_projected(bits(kb[b, : ref.shape[0]]), ref)
        assert st["kb_bit_equal_to_rne"] >= 0.99, st
        assert torch.all(kb[b, ref.shape[0]:] == 7.0)
    # refresh only the trailing block of each sequence after zeroing it
    last = [-(-L_ // B) - 1 for L_ in lens]
    for b in range(n):
        kb[b, last[b]] = 0
    before = kb.clone()
    for b, L_ in enumerate(lens):
        sgqa.index_build_from_keys(shape, K[b], wkt, kb[b], [L_], last[b], last[b] + 1)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        ref = oracle.index_build_from_keys(bits(K[b, last[b] * B: L_]), bits(wkt), B)
        parity.check_kb_projected(bits(kb[b, last[b]:last[b] + 1]), ref)
        mask = torch.ones(nblk, dtype=torch.bool, device=DEV)
        mask[last[b]] = False
        assert torch.equal(kb[b][mask], before[b][mask])


def test_tiny_index_decode_loop_trailing_block(tiny):
    """A decode loop's index maintenance: three sequences grow by one token per step across
    block boundaries (8, 517 and 1007 tokens at the start), and each step refreshes only the
    sequence's trailing block, from the proxy keys (sgqa_index_build) and from the keys
    (sgqa_index_build_from_keys).  After every step each sequence's index equals the oracle's
    build of its current length, and no other block changed."""
    shape = WL.shape
    B = shape.block_size
    lens = [8, 517, 1007]
    steps = 11
    n, Lmax = len(lens), max(lens) + steps
    kp = torch.zeros((n, Lmax, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    K = torch.zeros((n, Lmax) + tuple(tiny["K"].shape[1:]), dtype=torch.bfloat16, device=DEV)
    for b in range(n):
        kp[b] = tiny["kp"][:Lmax].roll(shifts=131 * b, dims=0)
        K[b] = tiny["K"][:Lmax].roll(shifts=131 * b, dims=0)
    wkt = _w_kt(WL, 3)
    nblk = -(-Lmax // B)
    kb = torch.full((n, nblk, shape.proxy_dim), 7.0, dtype=torch.bfloat16, device=DEV)
    kf = torch.full_like(kb, 7.0)
    sgqa.index_build(shape, kp, kb, lens)
    sgqa.index_build_from_keys(shape, K, wkt, kf, lens)
    for step in range(steps):
        lens = [L_ + 1 for L_ in lens]
        before, before_f = kb.clone(), kf.clone()
        last = [-(-L_ // B) - 1 for L_ in lens]
        for b, L_ in enumerate(lens):
            sgqa.index_build(shape, kp[b], kb[b], [L_], last[b], last[b] + 1)
            sgqa.index_build_from_keys(shape, K[b], wkt, kf[b], [L_], last[b], last[b] + 1)
        torch.cuda.synchronize()
        for b, L_ in enumerate(lens):
            nb = last[b] + 1
            st = parity.check_kb(bits(kb[b, :nb]), oracle.index_build(bits(kp[b, :L_]), B))
            assert st["kb_bit_equal_to_rne"] >= 0.999, (step, b, st)
            ref = oracle.index_build_from_keys(bits(K[b, last[b] * B: L_]), bits(wkt), B)
            parity.check_kb_projected(bits(kf[b, last[b]:nb]), ref)
            mask = torch.ones(nblk, dtype=torch.bool, device=DEV)
            mask[last[b]] = False
            assert torch.equal(kb[b][mask], before[b][mask]), (step, b)
            assert torch.equal(kf[b][mask], before_f[b][mask]), (step, b)
            assert torch.all(kb[b, nb:] == 7.0) and torch.all(kf[b, nb:] == 7.0)
    say(f"index decode loop: {steps} steps, lengths now {lens}")


@pytest.mark.parametrize("B", [8, 16])
def test_index_from_keys_odd_width(B):
    """Fused index maintenance where the key width (1 KV head x 192) is not a multiple of the
    kernel's 128-column step (a 64-column last step), proxy 64, for B = 8 and 16 (two row
    groups per step); then a rebuild of blocks [70, 200), which starts inside a workgroup's
    range of a full build, must give the same bits as the full build."""
    from long_context_sparse_18_amd.configs import LayerShape
    shape = LayerShape(num_q_heads=8, num_kv_heads=1, head_dim=192, proxy_dim=64,
                       block_size=B, topk_blocks=16)
    lens = [3001, 1024, 37]
    n, Lmax = len(lens), max(lens)
    g = torch.Generator(device=DEV).manual_seed(21)
    K = torch.randn((n, Lmax, 1, 192), generator=g, device=DEV).to(torch.bfloat16)
    wkt = (torch.randn((64, 192), generator=g, device=DEV) / 14).to(torch.bfloat16)
    nblk = -(-Lmax // B)
    kb = torch.full((n, nblk, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    sgqa.index_build_from_keys(shape, K, wkt, kb, lens)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        ref = oracle.index_build_from_keys(bits(K[b, :L_]), bits(wkt), B)
        st = parity.check_kb_projected(bits(kb[b, : ref.shape[0]]), ref)
        assert st["kb_bit_equal_to_rne"] >= 0.99, st
        assert torch.all(kb[b, ref.shape[0]:] == 7.0)
    full = kb.clone()
    kb[0, 70:200] = 0
    sgqa.index_build_from_keys(shape, K[0], wkt, kb[0], [lens[0]], 70, 200)
    torch.cuda.synchronize()
    assert torch.equal(kb, full)


def test_quantize_fp8_bit_exact():
    """Row quantisation to E4M3 codes and fp32 scales equals the oracle bit for bit, on rows of
    32, 64, 192 and 256 values spanning 2^-60 .. 2^60 in magnitude, with an all-zero row and
    rows that reach the subnormal codes."""
    g = torch.Generator().manual_seed(41)
    for cols in (32, 64, 192, 256):
        x = torch.randn((300, cols), generator=g) * torch.exp2(torch.randint(-60, 60, (300, 1),
                                                                               generator=g).float())
        x[3] = 0.0
        x[5, :] = x[5, :] * 1e-3  # small values next to one large one: subnormal codes
        x[5, 0] = 1.0
        xb = x.to(torch.bfloat16).to(DEV)
        codes = torch.empty(xb.shape, dtype=torch.uint8, device=DEV)
        scales = torch.empty(xb.shape[0], dtype=torch.float32, device=DEV)
        sgqa.quantize_fp8(xb, codes, scales)
        torch.cuda.synchronize()
        rc, rs = oracle.quantize_rows(bits(xb))
        assert np.array_equal(codes.cpu().numpy(), rc), cols
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32)), cols


def test_decode_fp8_mixed_lengths():
    """FP8 decode (index and K/V caches stored as E4M3 rows with fp32 scales) for 5 sequences
    of 1 .. 1024 tokens: codes bit-exact, selection and attention against the oracle on the
    dequantised values."""
    shape = dataclasses.replace(WL.shape, proxy_dim=64)
    wl = dataclasses.replace(WL, shape=shape)
    d = inputs.make_prefill(wl, 5, DEV)
    lens = [1, 9, 130, 1000, 1024]
    n, Lmax, B, k = len(lens), wl.L, shape.block_size, shape.topk_blocks
    K = d["K"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    V = d["V"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    kp = d["kp"].unsqueeze(0).expand(n, -1, -1).contiguous()
    Q = torch.stack([d["Q"][L_ - 1] for L_ in lens])
    G = torch.stack([d["G"][L_ - 1] for L_ in lens])
    qp = torch.stack([d["qp"][L_ - 1] for L_ in lens])
    kb = torch.empty((n, wl.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, kp, kb, lens)
    kbq = torch.empty(kb.shape, dtype=torch.uint8, device=DEV)
    kbs = torch.empty(kb.shape[:2], dtype=torch.float32, device=DEV)
    Kq = torch.empty(K.shape, dtype=torch.uint8, device=DEV)
    Vq = torch.empty(V.shape, dtype=torch.uint8, device=DEV)
    Ks = torch.empty(K.shape[:3], dtype=torch.float32, device=DEV)
    Vs = torch.empty(V.shape[:3], dtype=torch.float32, device=DEV)
    sgqa.quantize_fp8(kb, kbq, kbs)
    sgqa.quantize_fp8(K, Kq, Ks)
    sgqa.quantize_fp8(V, Vq, Vs)
    idx = torch.empty((n, k), dtype=torch.int32, device=DEV)
    sel = torch.empty((n, k), dtype=torch.float32, device=DEV)
    sgqa.indexer_topk_fp8(shape, qp, kbq, kbs, [L_ - 1 for L_ in lens], idx, sel)
    out = torch.empty_like(Q)
    lse = torch.empty((n, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.sparse_attn_decode_fp8(shape, Q, Kq, Vq, Ks, Vs, G, idx, lens, scale, out, lse)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows(bits(K[0]))
    assert np.array_equal(Kq[0].cpu().numpy(), rc) and np.array_equal(Ks[0].cpu().numpy(), rs)
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        c = int(t[0] // B)
        nb = -(-L_ // B)
        kb_deq = oracle.dequant_rows(kbq[b, :nb].cpu().numpy(), kbs[b, :nb].cpu().numpy())
        sc = oracle.scores(bits(qp[b:b + 1]), t, B, kb_deq, width=max(1, nb))
        ref = oracle.topk(sc, t, B, k)
        got = idx[b].cpu().numpy()
        parity.check_selection(got, sc[0], c, k, ref[0])
        parity.check_sel_scores(sel[b].cpu().numpy(), got, sc[0], c, k)
        toks = torch.from_numpy(oracle.token_set(got, B, L_ - 1)).to(DEV)
        kd = oracle.dequant_rows(Kq[b].index_select(0, toks).cpu().numpy(),
                                 Ks[b].index_select(0, toks).cpu().numpy())
        vd = oracle.dequant_rows(Vq[b].index_select(0, toks).cpu().numpy(),
                                 Vs[b].index_select(0, toks).cpu().numpy())
        o_ref, l_ref = oracle.attend_f64(bits(Q[b]), kd, vd, bits(G[b]), scale)
        parity.check_attention(bits(out[b:b + 1]), o_ref[None], lse[b:b + 1].cpu().numpy(),
                               l_ref[None])


def _backward_case(d, shape, q0: int, L: int, seed: int):
    """Forward on the GPU (index, top-k, attention with lse), then the backward for a seeded
    dout; returns the GPU gradients and the oracle's on the same selection."""
    B, k = shape.block_size, shape.topk_blocks
    Q, G = d["Q"][q0:], d["G"][q0:]
    T = Q.shape[0]
    kb = torch.empty((-(-L // B), shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, d["kp"][:L], kb, [L])
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, d["qp"][q0:], kb, [q0], idx)
    scale = 1.0 / math.sqrt(shape.head_dim)
    out = torch.empty_like(Q)
    lse = torch.empty((T, shape.num_q_heads), dtype=torch.float32, device=DEV)
    K, V = d["K"][:L], d["V"][:L]
    sgqa.sparse_attn_prefill(shape, Q, K, V, G, idx, q0, L, scale, out, lse)
    g = torch.Generator(device=DEV).manual_seed(seed)
    dout = torch.randn(Q.shape, generator=g, device=DEV).to(torch.bfloat16)
    grads = dict(dq=torch.empty(Q.shape, dtype=torch.float32, device=DEV),
                 dk=torch.empty(K.shape, dtype=torch.float32, device=DEV),
                 dv=torch.empty(V.shape, dtype=torch.float32, device=DEV),
                 dg=torch.empty(G.shape, dtype=torch.float32, device=DEV))
    sgqa.sparse_attn_backward(shape, Q, K, V, G, idx, q0, L, scale, lse, dout,
                              grads["dq"], grads["dk"], grads["dv"], grads["dg"])
    torch.cuda.synchronize()
    t = np.arange(q0, q0 + T, dtype=np.int64)
    ref = oracle.sparse_attention_backward(bits(Q), t, bits(K), bits(V), bits(G),
                                           idx.cpu().numpy(), B, scale, bits(dout))
    return grads, dict(zip(("dq", "dk", "dv", "dg"), ref)), (Q, K, V, G, idx, out, lse, dout)


@pytest.mark.parametrize("B,k,q0", [(8, 16, 0), (8, 4, 0), (1, 64, 0), (8, 16, 517), (16, 8, 100),
                                    (1, 2, 600)])
def test_tiny_backward(tiny, B, k, q0):
    """Fixed-selection backward on the tiny layer against the oracle: every dq, dK, dV and
    dgate element, sparse and dense rows, B in {1, 8, 16}, a chunk starting mid-block.  dq
    runs on the resident schedule except for (B 1, k 2, from row 600), whose histories span
    more ranges than it takes (the one-pass dq kernel).  A
    second call that sweeps the query rows for dK / dV in phases of 32 (then 96) rows gives
    identical bits: every sum keeps one fixed order.  With the forward output given (D from
    dout . out) dq, dK and dgate meet the same bar and dV keeps its bits."""
    shape = with_selection(WL.shape, B, k)
    grads, ref, args = _backward_case(tiny, shape, q0, WL.L, 7 + q0)
    st = {}
    for name in ("dq", "dk", "dv", "dg"):
        st.update(parity.check_grad(name, grads[name].cpu().numpy(), ref[name]))
    say(f"backward B={B} k={k} q0={q0}: {st}")
    Q, K, V, G, idx, out, lse, dout = args
    for row_slice in (32, 96):
        again = {n: torch.full_like(v, float("nan")) for n, v in grads.items()}
        sgqa.sparse_attn_backward(shape, Q, K, V, G, idx, q0, WL.L,
                                  1.0 / math.sqrt(shape.head_dim), lse, dout, again["dq"],
                                  again["dk"], again["dv"], again["dg"], dkdv_row_slice=row_slice)
        torch.cuda.synchronize()
        for n in grads:
            assert torch.equal(grads[n], again[n]), (n, row_slice)
    # D from the forward's bf16 output: one dq sweep; dV does not involve D, so its bits stay
    fo = {n: torch.full_like(v, float("nan")) for n, v in grads.items()}
    sgqa.sparse_attn_backward(shape, Q, K, V, G, idx, q0, WL.L, 1.0 / math.sqrt(shape.head_dim),
                              lse, dout, fo["dq"], fo["dk"], fo["dv"], fo["dg"], out=out)
    torch.cuda.synchronize()
    assert torch.equal(fo["dv"], grads["dv"])
    st = {}
    for name in ("dq", "dk", "dg"):
        st.update(parity.check_grad(name, fo[name].cpu().numpy(), ref[name]))
    say(f"backward with out B={B} k={k} q0={q0}: {st}")


@pytest.mark.gpu
def test_tiny_backward_beside_other_kernels(tiny):
    """The resident dq and dK / dV schedules wait on each other's progress only to order the work
    for the caches: with matrix products running on a second stream as the backward starts (so
    some of its workgroups start late and waiting waves run into their bound), every gradient bit
    is the same as in a call run alone."""
    shape = with_selection(WL.shape, 8, 16)
    grads, _, args = _backward_case(tiny, shape, 0, WL.L, 11)
    Q, K, V, G, idx, out, lse, dout = args
    side = torch.cuda.Stream(DEV)
    x = torch.randn((4096, 4096), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    again = {n: torch.full_like(v, float("nan")) for n, v in grads.items()}
    with torch.cuda.stream(side):
        for _ in range(4):
            y = torch.mm(x, x)
    sgqa.sparse_attn_backward(shape, Q, K, V, G, idx, 0, WL.L, 1.0 / math.sqrt(shape.head_dim),
                              lse, dout, again["dq"], again["dk"], again["dv"], again["dg"])
    torch.cuda.synchronize()
    del y
    for n in grads:
        assert torch.equal(grads[n], again[n]), n


def test_peak_probes():
    """The machine-peak probes compute what they state: every MFMA-probe wave reports
    2048 * iters (37 waves: a partial last workgroup), and the read probe's partial sums add
    up to the buffer's 32-bit word sum mod 2^32, for a buffer that leaves a ragged tail over
    the grid stride and for a single 16-byte word."""
    sink = torch.full((37,), -1.0, dtype=torch.float32, device=DEV)
    probe.probe_mfma_bf16(sink, 100)
    torch.cuda.synchronize()
    assert torch.all(sink == 204800.0), sink
    g = torch.Generator(device=DEV).manual_seed(3)
    for words in (1 << 20, 4):
        buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), dtype=torch.int32, device=DEV,
                            generator=g)
        part = torch.empty(96, dtype=torch.int32, device=DEV)
        probe.probe_read(buf, part)
        torch.cuda.synchronize()
        want = int(buf.to(torch.int64).sum().item()) & 0xFFFFFFFF
        got = int(part.to(torch.int64).sum().item()) & 0xFFFFFFFF
        assert got == want, (words, got, want)
    # gathers of 384-byte rows (and of 16-byte rows) in a random order, with repeats
    for row_words, n in ((96, 5000), (4, 777)):
        table = torch.randint(-2 ** 31, 2 ** 31 - 1, (1000, row_words), dtype=torch.int32,
                              device=DEV, generator=g)
        idx = torch.randint(0, 1000, (n,), dtype=torch.int32, device=DEV, generator=g)
        part = torch.empty(96, dtype=torch.int32, device=DEV)
        probe.probe_gather(table, idx, part)
        torch.cuda.synchronize()
        want = int(table.index_select(0, idx.long()).to(torch.int64).sum().item()) & 0xFFFFFFFF
        got = int(part.to(torch.int64).sum().item()) & 0xFFFFFFFF
        assert got == want, (row_words, n, got, want)
