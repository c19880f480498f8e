"""GPU parity on layer shapes beyond the two workloads, each against the oracle on every row of
a 1024-token sequence: head_dim 128; 1, 2, 4 and 8 query heads per KV group; 3 KV groups
(which do not divide the 8 XCDs, so the kernels take their other workgroup mapping) and 8;
proxy widths 32 to 512; B from 2 to 16.  Stages: index, top-k and attention of the prefill,
decode for three sequences of different lengths (also with FP8 storage), sliding-window
attention, the index from the keys, and the fixed-selection backward."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from gpu_layer import check_prefill_rows, run_prefill, say
from long_context_sparse_18_amd import inputs, sgqa
from long_context_sparse_18_amd.configs import LayerShape, Workload
from long_context_sparse_18_amd.inputs import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (Hq, Hkv, d, P, B, k)
SHAPES = [
    LayerShape(8, 2, 128, 64, 8, 16),
    LayerShape(16, 2, 64, 512, 8, 16),
    LayerShape(32, 4, 192, 128, 16, 8),
    LayerShape(4, 4, 64, 32, 4, 32),
    LayerShape(6, 3, 64, 32, 8, 16),
    LayerShape(16, 8, 128, 256, 2, 64),
]


def _id(s):
    return f"hq{s.num_q_heads}-hkv{s.num_kv_heads}-d{s.head_dim}-p{s.proxy_dim}-b{s.block_size}-k{s.topk_blocks}"


@pytest.fixture(scope="module", params=SHAPES, ids=_id)
def case(request):
    shape = request.param
    wl = Workload("shape-1k", shape, nseq=1, T=1024, L=1024, q_start=0)
    say(f"shapes: generating {_id(shape)}")
    d = inputs.make_prefill(wl, 5, DEV)
    return wl, d, (bits(d["K"]), bits(d["V"]))


@pytest.mark.parametrize("sliced", [False, True], ids=["one-pass", "history-sliced"])
def test_shape_prefill_every_row(case, sliced):
    wl, d, host = case
    ws = None
    if sliced:  # with a workspace each row's history is attended in slices
        ws = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, wl.shape, 1, wl.T, wl.L),
                         dtype=torch.uint8, device=DEV)
    res = run_prefill(wl.shape, d, 0, wl.L, attn_workspace=ws)
    rows = np.arange(wl.T)
    st = check_prefill_rows(wl.shape, d, res, 0, rows, host_cache=host)
    say(f"shapes {_id(wl.shape)} prefill (sliced={sliced}): {st}")
    assert st["exact_iso"] >= len(rows) - 2


def test_shape_decode(case):
    wl, d, host = case
    shape = wl.shape
    B, k = shape.block_size, shape.topk_blocks
    lens = [1024, 700, 129]
    n = len(lens)
    K = d["K"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    V = d["V"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    kp = d["kp"].unsqueeze(0).expand(n, -1, -1).contiguous()
    Q = torch.stack([d["Q"][L_ - 1] for L_ in lens])
    G = torch.stack([d["G"][L_ - 1] for L_ in lens])
    qp = torch.stack([d["qp"][L_ - 1] for L_ in lens]).unsqueeze(1)
    kb = torch.empty((n, wl.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, kp, kb, lens)
    idx = torch.empty((n, 1, k), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1 for L_ in lens], idx)
    out = torch.empty_like(Q)
    lse = torch.empty((n, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.sparse_attn_decode(shape, Q, K, V, G, idx.view(n, -1), lens, scale, out, lse)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        nb = -(-L_ // B)
        sc = oracle.scores(bits(qp[b]), t, B, parity.widen(bits(kb[b, :nb])), width=max(1, nb))
        ref = oracle.topk(sc, t, B, k)
        got = idx[b, 0].cpu().numpy()
        parity.check_selection(got, sc[0], int(t[0] // B), k, ref[0])
        o_ref, l_ref = oracle.sparse_attention(bits(Q[b:b + 1]), t, host[0][:L_], host[1][:L_],
                                               bits(G[b:b + 1]), got[None, :], B, scale)
        parity.check_attention(bits(out[b:b + 1]), o_ref, lse[b:b + 1].cpu().numpy(), l_ref)


def test_shape_sliding_window(case):
    wl, d, host = case
    shape = wl.shape
    window = 100
    out = torch.empty_like(d["Q"])
    lse = torch.empty((wl.T, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.swa_prefill(shape, d["Q"], d["K"], d["V"], d["G"], 0, wl.L, window, scale, out, lse)
    torch.cuda.synchronize()
    t = np.arange(wl.T)
    o_ref, l_ref = oracle.window_attention(bits(d["Q"]), t, host[0], host[1], bits(d["G"]),
                                           window, scale)
    parity.check_attention(bits(out), o_ref, lse.cpu().numpy(), l_ref)


def test_shape_index_from_keys(case):
    wl, d, host = case
    shape = wl.shape
    wkt = inputs.proxy_weights(wl, 5, DEV)[1].t().contiguous().to(torch.bfloat16)
    kb = torch.empty((wl.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build_from_keys(shape, d["K"], wkt, kb, [wl.L])
    torch.cuda.synchronize()
    ref = oracle.index_build_from_keys(host[0], bits(wkt), shape.block_size)
    st = parity.check_kb_projected(bits(kb), ref)
    assert st["kb_bit_equal_to_rne"] >= 0.99, st


def test_shape_backward(case):
    wl, d, host = case
    shape = wl.shape
    B = shape.block_size
    res = run_prefill(shape, d, 0, wl.L)
    g = torch.Generator(device=DEV).manual_seed(17)
    dout = torch.randn(d["Q"].shape, generator=g, device=DEV).to(torch.bfloat16)
    grads = dict(dq=torch.empty(d["Q"].shape, dtype=torch.float32, device=DEV),
                 dk=torch.empty(d["K"].shape, dtype=torch.float32, device=DEV),
                 dv=torch.empty(d["V"].shape, dtype=torch.float32, device=DEV),
                 dg=torch.empty(d["G"].shape, dtype=torch.float32, device=DEV))
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.sparse_attn_backward(shape, d["Q"], d["K"], d["V"], d["G"], res["idx"], 0, wl.L, scale,
                              res["lse"], dout, grads["dq"], grads["dk"], grads["dv"], grads["dg"])
    torch.cuda.synchronize()
    t = np.arange(wl.T, dtype=np.int64)
    ref = oracle.sparse_attention_backward(bits(d["Q"]), t, host[0], host[1], bits(d["G"]),
                                           res["idx"].cpu().numpy(), B, scale, bits(dout))
    st = {}
    for name, r in zip(("dq", "dk", "dv", "dg"), ref):
        st.update(parity.check_grad(name, grads[name].cpu().numpy(), r))
    say(f"shapes {_id(shape)} backward: {st}")
    # D from the forward output: dq, dK and dgate meet the same bar, dV keeps its bits
    fo = {n: torch.full_like(v, float("nan")) for n, v in grads.items()}
    sgqa.sparse_attn_backward(shape, d["Q"], d["K"], d["V"], d["G"], res["idx"], 0, wl.L, scale,
                              res["lse"], dout, fo["dq"], fo["dk"], fo["dv"], fo["dg"],
                              out=res["out"])
    torch.cuda.synchronize()
    assert torch.equal(fo["dv"], grads["dv"])
    st = {}
    for name, r in zip(("dq", "dk", "dv", "dg"), ref):
        if name != "dv":
            st.update(parity.check_grad(name, fo[name].cpu().numpy(), r))
    say(f"shapes {_id(shape)} backward with out: {st}")


def test_shape_decode_fp8(case):
    """The FP8-storage decode path (E4M3 rows with one fp32 scale each for the index and the
    K/V caches) against the oracle on the dequantised values."""
    wl, d, host = case
    shape = wl.shape
    if shape.proxy_dim not in (64, 128, 256, 512):
        pytest.skip("the FP8 index takes proxy widths 64 to 512 (the API reports 32 unsupported)")
    B, k = shape.block_size, shape.topk_blocks
    lens = [1024, 333]
    n = len(lens)
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
    sgqa.indexer_topk_fp8(shape, qp, kbq, kbs, [L_ - 1 for L_ in lens], idx)
    out = torch.empty_like(Q)
    lse = torch.empty((n, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.sparse_attn_decode_fp8(shape, Q, Kq, Vq, Ks, Vs, G, idx, lens, scale, out, lse)
    torch.cuda.synchronize()
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        nb = -(-L_ // B)
        kb_deq = oracle.dequant_rows(kbq[b, :nb].cpu().numpy(), kbs[b, :nb].cpu().numpy())
        sc = oracle.scores(bits(qp[b:b + 1]), t, B, kb_deq, width=max(1, nb))
        ref = oracle.topk(sc, t, B, k)
        got = idx[b].cpu().numpy()
        parity.check_selection(got, sc[0], int(t[0] // B), k, ref[0])
        toks = torch.from_numpy(oracle.token_set(got, B, L_ - 1)).to(DEV)
        kd = oracle.dequant_rows(Kq[b].index_select(0, toks).cpu().numpy(),
                                 Ks[b].index_select(0, toks).cpu().numpy())
        vd = oracle.dequant_rows(Vq[b].index_select(0, toks).cpu().numpy(),
                                 Vs[b].index_select(0, toks).cpu().numpy())
        o_ref, l_ref = oracle.attend_f64(bits(Q[b]), kd, vd, bits(G[b]), scale)
        parity.check_attention(bits(out[b:b + 1]), o_ref[None], lse[b:b + 1].cpu().numpy(),
                               l_ref[None])


def test_decode_largest_batch():
    """Decode for the largest batch the API takes (64 sequences), caches of 1 to 1024 tokens
    on the tiny layer: every sequence's selection and output against the oracle."""
    from long_context_sparse_18_amd import WORKLOADS
    wl = WORKLOADS[0]
    shape = wl.shape
    B, k = shape.block_size, shape.topk_blocks
    d = inputs.make_prefill(wl, 9, DEV)
    lens = [1 + (37 * i) % 1024 for i in range(64)]
    lens[0], lens[1] = 1024, 1
    n = len(lens)
    K = d["K"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    V = d["V"].unsqueeze(0).expand(n, -1, -1, -1).contiguous()
    kp = d["kp"].unsqueeze(0).expand(n, -1, -1).contiguous()
    Q = torch.stack([d["Q"][L_ - 1] for L_ in lens])
    G = torch.stack([d["G"][L_ - 1] for L_ in lens])
    qp = torch.stack([d["qp"][L_ - 1] for L_ in lens]).unsqueeze(1)
    kb = torch.empty((n, wl.nblk, shape.proxy_dim), dtype=torch.bfloat16, device=DEV)
    sgqa.index_build(shape, kp, kb, lens)
    idx = torch.empty((n, 1, k), dtype=torch.int32, device=DEV)
    sgqa.indexer_topk(shape, qp, kb, [L_ - 1 for L_ in lens], idx)
    out = torch.empty_like(Q)
    lse = torch.empty((n, shape.num_q_heads), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(shape.head_dim)
    sgqa.sparse_attn_decode(shape, Q, K, V, G, idx.view(n, -1), lens, scale, out, lse)
    torch.cuda.synchronize()
    Kb, Vb = bits(d["K"]), bits(d["V"])
    for b, L_ in enumerate(lens):
        t = np.array([L_ - 1])
        nb = -(-L_ // B)
        sc = oracle.scores(bits(qp[b]), t, B, parity.widen(bits(kb[b, :nb])), width=max(1, nb))
        ref = oracle.topk(sc, t, B, k)
        got = idx[b, 0].cpu().numpy()
        parity.check_selection(got, sc[0], int(t[0] // B), k, ref[0])
        o_ref, l_ref = oracle.sparse_attention(bits(Q[b:b + 1]), t, Kb[:L_], Vb[:L_],
                                               bits(G[b:b + 1]), got[None, :], B, scale)
        parity.check_attention(bits(out[b:b + 1]), o_ref, lse[b:b + 1].cpu().numpy(), l_ref)


def test_prefill_largest_selection_32k():
    """The largest selection the API takes at B = 8 (k = 4 096 blocks = 32 768 tokens) on the
    32K prefill at the real layer shape, where every query attends its whole causal history:
    sampled rows (block edges, the k*B edge, random rows) against the oracle."""
    from long_context_sparse_18_amd import WORKLOADS
    from long_context_sparse_18_amd.configs import with_selection
    wl = WORKLOADS[1]
    shape = with_selection(wl.shape, 8, 4096)
    say("shapes: 32K prefill at k = 4096")
    d = inputs.make_prefill(wl, 13, DEV)
    res = run_prefill(shape, d, 0, wl.L)
    rows = parity.stratified_rows(0, wl.T, 8, 4096, 16, 3)
    st = check_prefill_rows(shape, d, res, 0, rows)
    say(f"shapes: 32K k=4096: {st}")
    assert st["exact_iso"] == st["rows"]
    del d, res
    torch.cuda.empty_cache()
