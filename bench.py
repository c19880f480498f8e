"""Benchmark of the Sparse GQA full-attention layer on one MI355X.

A step is one pass of the whole layer over the 131 072-token prefill workload
(64 query heads, 4 KV heads, d 192, proxy 256, blocks of 8, top-512 blocks):
sgqa_index_build over every block, sgqa_indexer_topk for every query, and
sgqa_sparse_attn_prefill.  Inputs are synthetic and already resident in HBM.
The decode workload (16 sequences x 1 048 576 cached tokens, one query each:
sgqa_indexer_topk + sgqa_sparse_attn_decode on a prebuilt index) is timed on the
same line under "decode".  Kernel durations come from HIP events recorded on
the stream the kernels run on.  The CPU baseline is the fp64 oracle on a sample
of query rows, timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sparse-GQA prefill tokens/s/layer @128K; decode µs/layer @1M; % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def measured_traffic(name: str):
    """HBM bytes per launch from a committed rocprofv3 summary, or None when the kernel's
    sources changed since the counters were taken (their hash no longer matches)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest()[:16] != rec["source_sha"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def attended_pairs(q_start: int, T: int, B: int, k: int) -> int:
    """Sum over queries of |U_t| (tokens attended), from the selection rule."""
    total = 0
    for t in range(q_start, q_start + T):
        c = t // B
        total += t + 1 if c <= k - 1 else (k - 1) * B + (t % B) + 1
    return total


def scored_pairs(q_start: int, T: int, B: int) -> int:
    return sum(t // B for t in range(q_start, q_start + T))


PREFILL_CHUNKS = 1  # row ranges of the layer step (one stream; see layer.py)


def prefill_launches(wl) -> str:
    """How one sgqa_sparse_attn_prefill call over all rows of the workload is dispatched: every
    row's history spans at most 16 ranges of 5k blocks, so the call is one fill kernel and one
    persistent launch of the resident workgroups (2 of 4 waves per CU at 256 registers per
    wave), each XCD's 256 waves taking batches of 256 rows of its KV group through the ranges."""
    s = wl.shape
    W = 5 * s.topk_blocks
    per_batch = 8 // s.num_kv_heads * 256
    batches = -(-wl.T // per_batch)
    ranges = ((wl.q_start + wl.T - 1) // s.block_size) // W + 1
    return (f"one sgqa_sparse_attn_prefill call over all {wl.T} rows: a fill kernel, then one "
            f"persistent launch of 512 workgroups taking {batches} batches of {per_batch} rows "
            f"per KV group through up to {ranges} history ranges of {W} blocks")


def bench_prefill(steps: int, warmup: int):
    import torch
    from long_context_sparse_18_amd import WORKLOADS, inputs, layer, sgqa

    wl = WORKLOADS[2]
    s = wl.shape
    dev = torch.device("cuda:0")
    log(f"prefill: generating {wl.name}")
    d = inputs.make_prefill(wl, 2, dev)
    kb = torch.empty((wl.nblk, s.proxy_dim), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((wl.T, s.topk_blocks), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["Q"])
    lse = torch.empty((wl.T, s.num_q_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, s, 1, wl.T, wl.L),
                     dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, s, 1, wl.T, wl.L),
                          dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(s.head_dim)
    stream = torch.cuda.current_stream(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(marks):
        marks.append(ev())
        sgqa.index_build(s, d["kp"], kb, [wl.L], stream=stream)
        marks.append(ev())
        sgqa.indexer_topk(s, d["qp"], kb, [wl.q_start], idx, workspace=ws, stream=stream)
        marks.append(ev())
        sgqa.sparse_attn_prefill(s, d["Q"], d["K"], d["V"], d["G"], idx, wl.q_start, wl.L, scale,
                                 out, lse, workspace=ws_attn, stream=stream)
        marks.append(ev())

    # the timed step: the layer's own schedule on one stream (index build, selections, sparse
    # attention; same calls, same result bits)
    def layer_step():
        layer.prefill_layer(s, d, wl.q_start, wl.L, scale, kb, idx, out, lse, ws, ws_attn,
                            chunks=PREFILL_CHUNKS, stream=stream)

    for _ in range(warmup):
        layer_step()
    torch.cuda.synchronize()
    log(f"prefill: timing {steps} steps")
    t0 = ev()
    step_marks = [t0]
    for _ in range(steps):
        layer_step()
        step_marks.append(ev())
    t1 = step_marks[-1]
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    step_ms = sorted(step_marks[i].elapsed_time(step_marks[i + 1]) for i in range(steps))
    median_ms = step_ms[len(step_ms) // 2]
    # the stage times: the same stages one after the other on one stream
    step([])
    marks = []
    for _ in range(steps):
        step(marks)
    torch.cuda.synchronize()
    per = [[marks[4 * i + j].elapsed_time(marks[4 * i + j + 1]) for j in range(3)]
           for i in range(steps)]
    build_ms = sum(p[0] for p in per) / steps
    topk_ms = sum(p[1] for p in per) / steps
    attn_ms = sum(p[2] for p in per) / steps
    attn_ms_median = sorted(p[2] for p in per)[steps // 2]
    # the index build alone, back to back (one stage mark is too coarse for ~20 us)
    a0, a1 = ev(), None
    for _ in range(steps * 10):
        sgqa.index_build(s, d["kp"], kb, [wl.L], stream=stream)
    a1 = ev()
    torch.cuda.synchronize()
    build_loop_ms = a0.elapsed_time(a1) / (steps * 10)
    build_bytes = wl.L * s.proxy_dim * 2 + wl.nblk * s.proxy_dim * 2
    index_build = {"ms": build_loop_ms, "algorithmic_bytes": build_bytes,
                   "GBps": build_bytes / (build_loop_ms / 1e3) / 1e9,
                   "hbm_frac": build_bytes / (build_loop_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                   "traffic": measured_traffic("index_build_128k"),
                   "kernel": "k_index_build<8>",
                   "timing": f"{steps * 10} calls back to back, HIP events on the stream"}
    pairs = attended_pairs(wl.q_start, wl.T, s.block_size, s.topk_blocks)
    flops = 4 * s.head_dim * s.num_q_heads * pairs
    # algorithmic bytes of the attention launch: every attended (query, token) pair reads that
    # token's K and V rows of all KV heads; plus q, gate, idx in and out, lse out
    gather_bytes = pairs * s.num_kv_heads * s.head_dim * 2 * 2
    io_bytes = wl.T * (2 * s.num_q_heads * s.head_dim * 2 + s.num_q_heads * (2 + 4)
                       + s.topk_blocks * 4)
    # the sibling layer type on the same inputs: gated sliding-window attention, window 512
    W = 512
    swa_out = torch.empty_like(out)  # out keeps the sparse forward's output for the backward
    sgqa.swa_prefill(s, d["Q"], d["K"], d["V"], d["G"], wl.q_start, wl.L, W, scale, swa_out,
                     stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        sgqa.swa_prefill(s, d["Q"], d["K"], d["V"], d["G"], wl.q_start, wl.L, W, scale, swa_out,
                         stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    swa_ms = a.elapsed_time(b) / steps
    swa_pairs = sum(min(W, t + 1) for t in range(wl.q_start, wl.q_start + wl.T))
    swa = {"window": W, "ms": swa_ms, "tokens_per_s": wl.T / (swa_ms / 1e3),
           "tflops": 4 * s.head_dim * s.num_q_heads * swa_pairs / (swa_ms / 1e3) / 1e12}
    # index maintenance straight from the keys (no proxy-key tensor): every block of the
    # 128K cache, mean key projected by W^T [P, Hkv*d]
    wkt = inputs.proxy_weights(wl, 2, dev)[1].t().contiguous().to(torch.bfloat16)
    kb_f = torch.empty_like(kb)
    sgqa.index_build_from_keys(s, d["K"], wkt, kb_f, [wl.L], stream=stream)
    a.record(stream)
    for _ in range(steps):
        sgqa.index_build_from_keys(s, d["K"], wkt, kb_f, [wl.L], stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    fk_ms = a.elapsed_time(b) / steps
    width = s.num_kv_heads * s.head_dim
    fk_bytes = wl.L * width * 2 + wl.nblk * s.proxy_dim * 2 + s.proxy_dim * width * 2
    fused_index = {"ms": fk_ms, "GBps": fk_bytes / (fk_ms / 1e3) / 1e9,
                   "hbm_frac": fk_bytes / (fk_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                   "algorithmic_bytes": fk_bytes,
                   "mfma_tflops": 2 * 2 * wl.nblk * width * s.proxy_dim / (fk_ms / 1e3) / 1e12}
    del kb_f
    # backward of the attention with this step's selection fixed (training), same inputs
    g = torch.Generator(device=dev).manual_seed(9)
    dout = torch.randn(d["Q"].shape, generator=g, device=dev).to(torch.bfloat16)
    dq = torch.empty(d["Q"].shape, dtype=torch.float32, device=dev)
    dk = torch.empty(d["K"].shape, dtype=torch.float32, device=dev)
    dv = torch.empty(d["V"].shape, dtype=torch.float32, device=dev)
    dg = torch.empty(d["G"].shape, dtype=torch.float32, device=dev)
    ws_b = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_BACKWARD, s, 1, wl.T, wl.L),
                       dtype=torch.uint8, device=dev)

    def bwd(fwd_out=None):
        sgqa.sparse_attn_backward(s, d["Q"], d["K"], d["V"], d["G"], idx, wl.q_start, wl.L, scale,
                                  lse, dout, dq, dk, dv, dg, workspace=ws_b, stream=stream,
                                  out=fwd_out)

    def time_bwd(fwd_out):
        bwd(fwd_out)
        a.record(stream)
        for _ in range(steps):
            bwd(fwd_out)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    bwd_ms = time_bwd(None)
    # (the variant that takes D from the forward output is experimental: its dq error on the
    # 128K rows sits at the gradient bound, so it is not timed here)
    backward = {"ms": bwd_ms, "tokens_per_s": wl.T / (bwd_ms / 1e3),
                "tflops_minimal": 10 * s.head_dim * s.num_q_heads * pairs / (bwd_ms / 1e3) / 1e12,
                "ratio_to_forward_attention": bwd_ms / attn_ms}
    del dout, dq, dk, dv, dg, ws_b, swa_out
    res = dict(wl=wl, total_ms=total_ms, ms_per_step=total_ms / steps, build_ms=build_ms, swa=swa,
               median_ms=median_ms, attn_ms_median=attn_ms_median, index_build=index_build,
               sequential_ms=sum(sum(p) for p in per) / steps,
               fused_index=fused_index, backward=backward,
               topk_ms=topk_ms, attn_ms=attn_ms, pairs=pairs, attn_flops=flops,
               gather_bytes=gather_bytes, attn_bytes=gather_bytes + io_bytes, data=d, kb=kb,
               idx=idx)
    return res


def bench_chunked(steps: int, warmup: int, cpu: bool):
    """Chunked prefill: 8192 new query tokens at positions 1 040 388 .. 1 048 579 of a
    1 048 580-token cache (131 072 candidate blocks for the last rows).  A step is the index
    rebuild of the blocks the chunk touched ([130048, 131073)), the indexer top-k of the 8192
    rows and their sparse attention, one after the other on one stream."""
    import torch
    from long_context_sparse_18_amd import WORKLOADS, inputs, sgqa

    wl = WORKLOADS[4]
    s = wl.shape
    dev = torch.device("cuda:0")
    log(f"chunked prefill: generating {wl.name}")
    d = inputs.make_prefill(wl, 4, dev)
    kb = torch.empty((wl.nblk, s.proxy_dim), dtype=torch.bfloat16, device=dev)
    sgqa.index_build(s, d["kp"], kb, [wl.L])  # the history's index, built before the chunk
    blk0 = wl.q_start // s.block_size
    idx = torch.empty((wl.T, s.topk_blocks), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["Q"])
    lse = torch.empty((wl.T, s.num_q_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, s, 1, wl.T, wl.L),
                     dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_PREFILL, s, 1, wl.T, wl.L),
                          dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(s.head_dim)
    stream = torch.cuda.current_stream(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step():
        m = [ev()]
        sgqa.index_build(s, d["kp"], kb, [wl.L], blk_begin=blk0, stream=stream)
        m.append(ev())
        sgqa.indexer_topk(s, d["qp"], kb, [wl.q_start], idx, workspace=ws, stream=stream)
        m.append(ev())
        sgqa.sparse_attn_prefill(s, d["Q"], d["K"], d["V"], d["G"], idx, wl.q_start, wl.L, scale,
                                 out, lse, workspace=ws_attn, stream=stream)
        m.append(ev())
        return m

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = [step() for _ in range(steps)]
    torch.cuda.synchronize()
    per = [[m[j].elapsed_time(m[j + 1]) for j in range(3)] for m in marks]
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    build_ms, topk_ms, attn_ms = (med([p[j] for p in per]) for j in range(3))
    layer_ms = med([sum(p) for p in per])
    pairs = attended_pairs(wl.q_start, wl.T, s.block_size, s.topk_blocks)
    sc_pairs = scored_pairs(wl.q_start, wl.T, s.block_size)
    attn_flops = 4 * s.head_dim * s.num_q_heads * pairs
    res = {"workload": wl.name, "T": wl.T, "L": wl.L, "q_start": wl.q_start,
           "ms_per_step": layer_ms, "tokens_per_s": wl.T / (layer_ms / 1e3),
           "stages_ms": {"index_build_range": build_ms, "indexer_topk": topk_ms,
                         "sparse_attn_prefill": attn_ms},
           "indexer_share": (build_ms + topk_ms) / layer_ms,
           "attention_tflops": attn_flops / (attn_ms / 1e3) / 1e12,
           "indexer_tflops": 2 * s.proxy_dim * sc_pairs / (topk_ms / 1e3) / 1e12,
           "indexer_to_attention_flops": (2 * s.proxy_dim * sc_pairs) / attn_flops,
           "timing": f"median of {steps} steps, stages one after the other on one stream"}
    log(f"chunked prefill: {layer_ms:.2f} ms/step (build {build_ms:.3f}, topk {topk_ms:.3f}, "
        f"attn {attn_ms:.3f}) -> {res['tokens_per_s']:,.0f} tokens/s, indexer share "
        f"{res['indexer_share']:.3f}")
    if cpu:
        res["cpu_baseline"] = cpu_baseline_chunked(wl, d, rows=512)
        log(f"chunked prefill cpu baseline: {res['cpu_baseline']['sample']}")
    del d, kb, idx, out, lse, ws, ws_attn
    torch.cuda.empty_cache()
    return res


def time_decode_step(topk, attn, flush, stream, steps: int, warmup: int):
    """Median microseconds of one decode step (top-k then attention, back to back on the
    stream) and of its two calls.  Every step starts after a 512 MiB read, so no step starts
    with the caches warm.  The whole-step figure comes from steps with events only at their
    ends: an event recorded between the two calls leaves the GPU idle for ~6 us while the
    marker is processed, so the split comes from separate steps with that middle event."""
    import torch

    def run(mid: bool):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        m = torch.cuda.Event(enable_timing=True) if mid else None
        a.record(stream)
        topk()
        if mid:
            m.record(stream)
        attn()
        b.record(stream)
        return a, m, b

    for _ in range(warmup):
        flush.sum()
        run(True)
    torch.cuda.synchronize()
    whole, t_topk, t_attn = [], [], []
    for _ in range(steps):
        for mid in (False, True):
            flush.sum()
            a, m, b = run(mid)
            torch.cuda.synchronize()
            if mid:
                t_topk.append(a.elapsed_time(m) * 1e3)
                t_attn.append(m.elapsed_time(b) * 1e3)
            else:
                whole.append(a.elapsed_time(b) * 1e3)

    def median(v):
        return sorted(v)[len(v) // 2]

    return median(whole), median(t_topk), median(t_attn)


def bench_decode(steps: int, warmup: int, cpu: bool = False):
    import torch
    from long_context_sparse_18_amd import WORKLOADS, inputs, sgqa

    wl = WORKLOADS[3]
    s = wl.shape
    n = wl.nseq
    dev = torch.device("cuda:0")
    log("decode: generating 16 x 1M-token caches")
    d = inputs.make_decode(wl, 3, dev)
    kb = torch.empty((n, wl.nblk, s.proxy_dim), dtype=torch.bfloat16, device=dev)
    sgqa.index_build(s, d["kp"], kb, [wl.L] * n)
    idx = torch.empty((n, 1, s.topk_blocks), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["Q"])
    ws_topk = torch.empty(sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, s, n, 1, wl.L),
                          dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(sgqa.workspace_bytes(sgqa.OP_ATTN_DECODE, s, n, 1, wl.L),
                          dtype=torch.uint8, device=dev)
    # cold-cache protocol: read (not write) 512 MiB between steps, so no dirty lines are
    # left to be written back while the timed kernels run
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(s.head_dim)
    stream = torch.cuda.current_stream(dev)
    qp = d["qp"].unsqueeze(1)

    def topk():
        sgqa.indexer_topk(s, qp, kb, [wl.L - 1] * n, idx, workspace=ws_topk, stream=stream)

    def attn():
        sgqa.sparse_attn_decode(s, d["Q"], d["K"], d["V"], d["G"], idx.view(n, -1), [wl.L] * n,
                                scale, out, workspace=ws_attn, stream=stream)

    med, us_topk, us_attn = time_decode_step(topk, attn, flush, stream, steps, warmup)
    # algorithmic bytes: the whole index scan, the gathered K/V rows, and the small tensors
    per_seq = ((wl.L - 1) // s.block_size) * s.proxy_dim * 2 \
        + s.topk_blocks * s.block_size * s.num_kv_heads * s.head_dim * 2 * 2 \
        + (2 * s.num_q_heads * s.head_dim * 2 + s.proxy_dim * 2 + s.num_q_heads * 2
           + s.topk_blocks * 4)
    bytes_total = per_seq * n
    res = dict(us_median=med, us_topk=us_topk, us_attn=us_attn, bytes=bytes_total,
               gbs=bytes_total / (med * 1e-6) / 1e9)
    if cpu:
        log("decode: oracle on all 16 sequences")
        res["cpu_baseline"] = cpu_baseline_decode(wl, d, d["qp"], idx.shape)
        log(f"decode cpu baseline: {res['cpu_baseline']['sample']}")
    del d["kp"]
    torch.cuda.empty_cache()

    # the same step on FP8 storage (E4M3 rows with one fp32 scale each) of index and caches
    log("decode: quantising index and caches to FP8")
    kbq = torch.empty(kb.shape, dtype=torch.uint8, device=dev)
    kbs = torch.empty(kb.shape[:2], dtype=torch.float32, device=dev)
    sgqa.quantize_fp8(kb, kbq, kbs)
    del kb
    cq = {}
    for name in ("K", "V"):
        cq[name] = (torch.empty(d[name].shape, dtype=torch.uint8, device=dev),
                    torch.empty(d[name].shape[:3], dtype=torch.float32, device=dev))
        sgqa.quantize_fp8(d[name], *cq[name])
        del d[name]
    torch.cuda.empty_cache()
    idx8 = idx.view(n, -1)

    def topk8():
        sgqa.indexer_topk_fp8(s, d["qp"], kbq, kbs, [wl.L - 1] * n, idx8, workspace=ws_topk,
                              stream=stream)

    def attn8():
        sgqa.sparse_attn_decode_fp8(s, d["Q"], cq["K"][0], cq["V"][0], cq["K"][1], cq["V"][1],
                                    d["G"], idx8, [wl.L] * n, scale, out, workspace=ws_attn,
                                    stream=stream)

    med8, us_topk8, us_attn8 = time_decode_step(topk8, attn8, flush, stream, steps, warmup)
    c = (wl.L - 1) // s.block_size
    per_seq8 = c * (s.proxy_dim + 4) \
        + s.topk_blocks * s.block_size * s.num_kv_heads * (s.head_dim + 4) * 2 \
        + (2 * s.num_q_heads * s.head_dim * 2 + s.proxy_dim * 2 + s.num_q_heads * 2
           + s.topk_blocks * 4)
    res["fp8"] = dict(us_median=med8, us_topk=us_topk8, us_attn=us_attn8, bytes=per_seq8 * n,
                      gbs=per_seq8 * n / (med8 * 1e-6) / 1e9)
    return res


def bench_coverage():
    """Token coverage on the 32 768-token prefill: the share of the exact (dense) softmax
    mass that lands on the selected tokens, exp(lse_sparse - lse_dense), averaged over all
    (query, head); at B=8 with 512 blocks and at B=1 with 2048 tokens.  Also times index
    build + indexer top-k at both settings (the pages' 8x cost cut)."""
    import torch
    from long_context_sparse_18_amd import WORKLOADS, inputs, sgqa, with_selection

    wl = WORKLOADS[1]
    dev = torch.device("cuda:0")
    d = inputs.make_prefill(wl, 1, dev)
    scale = 1.0 / math.sqrt(wl.shape.head_dim)
    stream = torch.cuda.current_stream(dev)
    lses, times = {}, {}
    for tag, B, k in (("b8_k512", 8, 512), ("b1_k2048", 1, 2048), ("dense", 8, wl.L // 8)):
        s = with_selection(wl.shape, B, k)
        kb = torch.empty((-(-wl.L // B), s.proxy_dim), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((wl.T, k), dtype=torch.int32, device=dev)
        ws = torch.empty(sgqa.workspace_bytes(sgqa.OP_INDEXER_TOPK, s, 1, wl.T, wl.L),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(d["Q"])
        lse = torch.empty((wl.T, s.num_q_heads), dtype=torch.float32, device=dev)
        best = None
        for rep in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sgqa.index_build(s, d["kp"], kb, [wl.L], stream=stream)
            sgqa.indexer_topk(s, d["qp"], kb, [0], idx, workspace=ws, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        sgqa.sparse_attn_prefill(s, d["Q"], d["K"], d["V"], d["G"], idx, 0, wl.L, scale, out, lse,
                                 stream=stream)
        torch.cuda.synchronize()
        lses[tag] = lse
        times[tag] = best
        del kb, idx, ws, out
    res = {"workload": wl.name,
           "indexer_ms": {k_: round(v, 4) for k_, v in times.items() if k_ != "dense"},
           "indexer_cost_ratio_b1_over_b8": times["b1_k2048"] / times["b8_k512"],
           "pages_coverage_b8_k4096": 0.7806, "pages_coverage_b1_k2048": 0.7909}
    t = torch.arange(wl.T, device=dev)
    for tag, B, k in (("b8_k512", 8, 512), ("b1_k2048", 1, 2048)):
        cov = torch.exp((lses[tag] - lses["dense"]).double())
        res[f"coverage_{tag}"] = cov.mean().item()
        far = t >= k * B
        res[f"coverage_{tag}_t_ge_kB"] = cov[far].mean().item()
        # if the proxy scores carried no information about the logits, each attended token
        # would hold an equal share of the mass on average: E[cov_t] = |U_t| / (t + 1)
        c = t // B
        n_att = torch.where(c <= k - 1, t + 1, (k - 1) * B + t % B + 1)
        res[f"coverage_{tag}_if_uninformative"] = (n_att.double() / (t + 1)).mean().item()
    return res


def cpu_baseline(pre, rows: int, seed: int = 0, budget_s: float = 15.0):
    """The fp64 oracle on a sample of query rows of the same prefill workload: random rows in
    chunks of 256 until about `budget_s` seconds of oracle time or `rows` rows, whichever
    comes first, so the run stays bounded on a slow host."""
    import numpy as np
    import oracle
    from long_context_sparse_18_amd.inputs import bits

    wl = pre["wl"]
    s = wl.shape
    d = pre["data"]
    rng = np.random.default_rng(seed)
    order = rng.choice(wl.T, size=rows, replace=False).astype(np.int64)
    import torch
    kp = bits(d["kp"])
    K, V = bits(d["K"]), bits(d["V"])
    lib = oracle.load()
    t0 = time.perf_counter()
    kb = oracle.index_build(kp, s.block_size, lib=lib)
    t1 = time.perf_counter()
    done, t_sel, t_att = 0, 0.0, 0.0
    while done < rows and t_sel + t_att < budget_s:
        sel_rows = np.sort(order[done:done + 256])
        rt = torch.from_numpy(sel_rows).to(d["Q"].device)
        qp = bits(d["qp"].index_select(0, rt))
        q = bits(d["Q"].index_select(0, rt))
        g = bits(d["G"].index_select(0, rt))
        t = sel_rows + wl.q_start
        ta = time.perf_counter()
        sc = oracle.scores(qp, t, s.block_size, kb, width=max(1, int(t.max()) // s.block_size),
                           lib=lib)
        idx = oracle.topk(sc, t, s.block_size, s.topk_blocks, lib=lib)
        tb = time.perf_counter()
        oracle.sparse_attention(q, t, K, V, g, idx, s.block_size, 1.0 / math.sqrt(s.head_dim),
                                lib=lib)
        tc = time.perf_counter()
        t_sel += tb - ta
        t_att += tc - tb
        done += len(sel_rows)
    per_row = (t_sel + t_att) / done
    full_s = (t1 - t0) + per_row * wl.T
    host = host_description(lib)
    return {"value": wl.T / full_s, "unit": "tokens/s/layer", "cores": host["oracle_threads"],
            "kind": "oracle", "host": host, "extrapolated": True,
            "stages_s": {"index_build": t1 - t0, "scores_topk_per_row": t_sel / done,
                         "attention_per_row": t_att / done},
            "sample": (f"full index build ({t1 - t0:.2f} s) + {done} random query rows of the "
                       f"131072-token prefill (scores+sort {t_sel:.2f} s, attention "
                       f"{t_att:.2f} s), extrapolated to all rows")}


def host_description(lib=None) -> dict:
    """The host the oracle ran on: CPU model, logical CPUs, CPUs this process may use, the
    OpenMP setting and the threads the oracle's parallel loops actually ran on."""
    import oracle
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
            "oracle_threads": oracle.num_threads(lib)}


def cpu_baseline_chunked(wl, d, rows: int, seed: int = 0, budget_s: float = 20.0):
    """The fp64 oracle on the chunked prefill: the index rebuild of the blocks the chunk touched
    (timed in full), then scores + sort top-k and attention on random query rows in chunks of
    64 until about ``budget_s`` seconds or ``rows`` rows, extrapolated to all 8192 rows."""
    import numpy as np
    import oracle
    import torch
    from long_context_sparse_18_amd.inputs import bits

    s = wl.shape
    B = s.block_size
    lib = oracle.load()
    kp = bits(d["kp"])
    blk0 = wl.q_start // B
    kb = oracle.index_build(kp[: blk0 * B], B, lib=lib)  # the history, built before the chunk
    t0 = time.perf_counter()
    kb_new = oracle.index_build(kp[blk0 * B:], B, lib=lib)
    t1 = time.perf_counter()
    kb = np.concatenate([kb, kb_new])
    del kp
    K, V = bits(d["K"]), bits(d["V"])
    rng = np.random.default_rng(seed)
    order = rng.choice(wl.T, size=rows, replace=False).astype(np.int64)
    done, t_sel, t_att = 0, 0.0, 0.0
    while done < rows and t_sel + t_att < budget_s:
        sel_rows = np.sort(order[done:done + 64])
        rt = torch.from_numpy(sel_rows).to(d["Q"].device)
        t = sel_rows + wl.q_start
        qp = bits(d["qp"].index_select(0, rt))
        q, g = bits(d["Q"].index_select(0, rt)), bits(d["G"].index_select(0, rt))
        ta = time.perf_counter()
        sc = oracle.scores(qp, t, B, kb, width=int(t.max()) // B, lib=lib)
        idx = oracle.topk(sc, t, B, s.topk_blocks, lib=lib)
        tb = time.perf_counter()
        oracle.sparse_attention(q, t, K, V, g, idx, B, 1.0 / math.sqrt(s.head_dim), lib=lib)
        tc = time.perf_counter()
        t_sel += tb - ta
        t_att += tc - tb
        done += len(sel_rows)
    full_s = (t1 - t0) + (t_sel + t_att) / done * wl.T
    host = host_description(lib)
    return {"value": wl.T / full_s, "unit": "tokens/s/layer", "cores": host["oracle_threads"],
            "kind": "oracle", "host": host, "extrapolated": True,
            "stages_s": {"index_build_range": t1 - t0, "scores_topk_per_row": t_sel / done,
                         "attention_per_row": t_att / done},
            "sample": (f"index rebuild of blocks [{blk0}, {wl.nblk}) in full ({t1 - t0:.2f} s) "
                       f"+ {done} random query rows of the chunk (scores+sort {t_sel:.2f} s, "
                       f"attention {t_att:.2f} s), extrapolated to all {wl.T} rows")}


def cpu_baseline_decode(wl, d, qp, idx_shape) -> dict:
    """The fp64 oracle on the whole decode batch (16 sequences, one query each at t = L - 1):
    per sequence the scores over all 131 071 past blocks, the sort top-k and the attention,
    timed; the oracle's own index build of each sequence (untimed on the GPU path, where the
    index is precomputed) is timed separately."""
    import numpy as np
    import oracle
    from long_context_sparse_18_amd.inputs import bits

    s = wl.shape
    B = s.block_size
    lib = oracle.load()
    t = np.array([wl.L - 1], dtype=np.int64)
    c = (wl.L - 1) // B
    t_build = t_sel = t_att = 0.0
    for b in range(wl.nseq):
        kp = bits(d["kp"][b])
        ta = time.perf_counter()
        kb = oracle.index_build(kp, B, lib=lib)
        tb = time.perf_counter()
        del kp
        sc = oracle.scores(bits(qp[b:b + 1]), t, B, kb, width=c, lib=lib)
        sel = oracle.topk(sc, t, B, s.topk_blocks, lib=lib)
        tc = time.perf_counter()
        K, V = bits(d["K"][b]), bits(d["V"][b])
        td = time.perf_counter()
        oracle.sparse_attention(bits(d["Q"][b:b + 1]), t, K, V, bits(d["G"][b:b + 1]), sel, B,
                                1.0 / math.sqrt(s.head_dim), lib=lib)
        te = time.perf_counter()
        del K, V
        t_build += tb - ta
        t_sel += tc - tb
        t_att += te - td
    host = host_description(lib)
    us = (t_sel + t_att) * 1e6
    return {"value": us, "unit": "us/layer/batch", "cores": host["oracle_threads"],
            "kind": "oracle", "host": host, "extrapolated": False,
            "stages_s": {"scores_topk": t_sel, "attention": t_att,
                         "index_build_untimed_on_gpu": t_build},
            "sample": (f"all {wl.nseq} sequences of the 1 048 576-token decode in full: scores "
                       f"over 131 071 blocks + sort top-k {t_sel:.2f} s, attention {t_att:.2f} s "
                       f"(the oracle's index builds, {t_build:.2f} s, are outside the figure as "
                       f"the GPU's are)")}


def measure_peaks():
    """Measured machine peaks for the rooflines: dense bf16 MFMA (a loop of independent
    32x32x16 products in every SIMD) and streaming HBM reads (a 4 GiB buffer read once per
    pass), each checked against its closed-form result."""
    import torch
    from long_context_sparse_18_amd import probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves, iters = cus * 4 * 8, 4096
    sink = torch.empty(waves, dtype=torch.float32, device="cuda")
    probe.probe_mfma_bf16(sink, iters)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mfma_tflops = 0.0
    for _ in range(3):
        e0.record()
        probe.probe_mfma_bf16(sink, iters)
        e1.record()
        torch.cuda.synchronize()
        mfma_tflops = max(mfma_tflops,
                          waves * iters * 8 * 32768 / (e0.elapsed_time(e1) / 1e3) / 1e12)
    if not bool(torch.all(sink == 2048.0 * iters)):
        raise RuntimeError("MFMA probe returned a wrong result")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best = 0.0
    for blocks in (cus * 8, cus * 16, cus * 32):
        part = torch.empty(blocks, dtype=torch.int32, device="cuda")
        probe.probe_read(buf, part)
        e0.record()
        for _ in range(5):
            probe.probe_read(buf, part)
        e1.record()
        torch.cuda.synchronize()
        if int(part.to(torch.int64).sum().item()) & 0xFFFFFFFF != (nbytes // 4) & 0xFFFFFFFF:
            raise RuntimeError("read probe returned a wrong sum")
        best = max(best, 5 * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    # random gathers of 384-byte rows over 403 MB, the K/V footprint of the 128K layer
    rows, row_words, n = 1 << 20, 96, 1 << 26
    table = torch.ones((rows, row_words), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(0)
    idx = torch.randint(0, rows, (n,), dtype=torch.int32, device="cuda", generator=g)
    part = torch.empty(cus * 16, dtype=torch.int32, device="cuda")
    probe.probe_gather(table, idx, part)
    gather = 0.0
    for _ in range(3):
        e0.record()
        probe.probe_gather(table, idx, part)
        e1.record()
        torch.cuda.synchronize()
        gather = max(gather, n * row_words * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9)
    if int(part.to(torch.int64).sum().item()) & 0xFFFFFFFF != (n * row_words) & 0xFFFFFFFF:
        raise RuntimeError("gather probe returned a wrong sum")
    del table, idx
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": mfma_tflops, "hbm_read_GBps": best,
            "random_row_gather_GBps": gather,
            "gather_roofline_tflops": 16 * gather / 1e3,
            "method": f"{waves} waves x {iters} x 8 bf16 32x32x16 MFMA (best of 3); 4 GiB "
                      "streamed read, best of 8/16/32 workgroups per CU; 2^26 uniform random "
                      "384-byte rows of a 403 MB table (best of 3); the gather roofline is "
                      "16 flop per gathered byte (one K or V row feeds the 16 heads of its "
                      "group) times that gather rate"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3072)
    ap.add_argument("--no-coverage", action="store_true")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked prefill (8192 rows against 1M tokens)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="time only the decode workload (for profiling runs)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA / HBM-read peak probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run only the dense bf16 MFMA loop (calibrates the MFMA counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer is not sharded across GPUs here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_18_amd import probe, sgqa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(sgqa.lib_path()) or not os.path.exists(probe.lib_path()):
        from long_context_sparse_18_amd import build as _b
        _b.build()
    sgqa.load()
    probe.load()

    if args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 3 copies of 1 GiB")
        return
    if args.mfma_probe:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        waves, iters = cus * 4 * 8, 4096
        sink = torch.empty(waves, dtype=torch.float32, device="cuda")
        for _ in range(3):
            probe.probe_mfma_bf16(sink, iters)
        torch.cuda.synchronize()
        log(f"mfma probe: 3 x {waves} waves x {iters} x 8 bf16 32x32x16 products")
        return
    if args.no_prefill:
        dec = bench_decode(max(args.steps, 5), args.warmup)
        log(f"decode: {dec['us_median']:.1f} us/step (topk {dec['us_topk']:.1f}, attn "
            f"{dec['us_attn']:.1f}), {dec['gbs']:.0f} GB/s; FP8 storage "
            f"{dec['fp8']['us_median']:.1f} us/step (topk {dec['fp8']['us_topk']:.1f}, attn "
            f"{dec['fp8']['us_attn']:.1f}), {dec['fp8']['gbs']:.0f} GB/s")
        return

    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks()
        log(f"measured peaks: {peaks['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, "
            f"{peaks['hbm_read_GBps']:.0f} GB/s streamed HBM read, "
            f"{peaks['random_row_gather_GBps']:.0f} GB/s random 384-byte row gathers")
    pre = bench_prefill(args.steps, args.warmup)
    wl = pre["wl"]
    s = wl.shape
    tokens_per_s = wl.T / (pre["ms_per_step"] / 1e3)
    attn_tflops = pre["attn_flops"] / (pre["attn_ms"] / 1e3) / 1e12
    log(f"prefill: {pre['ms_per_step']:.2f} ms/step (stages one after the other "
        f"{pre['sequential_ms']:.2f}: build {pre['build_ms']:.3f}, topk {pre['topk_ms']:.3f}, "
        f"attn {pre['attn_ms']:.3f}) -> {tokens_per_s:,.0f} tokens/s, "
        f"attention {attn_tflops:.1f} TFLOP/s")
    log(f"sliding window: {pre['swa']['ms']:.3f} ms; index from keys: "
        f"{pre['fused_index']['ms']:.3f} ms ({pre['fused_index']['GBps']:.0f} GB/s); backward "
        f"{pre['backward']['ms']:.1f} ms ({pre['backward']['ratio_to_forward_attention']:.2f}x "
        f"the forward attention)")
    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle on up to {args.cpu_rows} rows (~15 s of oracle time)")
        cpu = cpu_baseline(pre, args.cpu_rows)
        log(f"cpu baseline: {cpu['sample']}")
    for key in ("data", "kb", "idx"):
        pre.pop(key, None)
    torch.cuda.empty_cache()
    cov = None
    if not args.no_coverage:
        log("coverage: 32K prefill at B=8/k=512, B=1/k=2048 and dense")
        cov = bench_coverage()
        log(f"coverage: {cov}")
        torch.cuda.empty_cache()
    chunked = None
    if not args.no_chunked:
        chunked = bench_chunked(max(args.steps // 2, 5), args.warmup, cpu=not args.no_cpu)
    dec = None
    if not args.no_decode:
        dec = bench_decode(max(args.steps, 5), args.warmup, cpu=not args.no_cpu)
        log(f"decode: {dec['us_median']:.1f} us/step (topk {dec['us_topk']:.1f}, attn "
            f"{dec['us_attn']:.1f}), {dec['gbs']:.0f} GB/s; FP8 storage "
            f"{dec['fp8']['us_median']:.1f} us/step (topk {dec['fp8']['us_topk']:.1f}, attn "
            f"{dec['fp8']['us_attn']:.1f}), {dec['fp8']['gbs']:.0f} GB/s")

    traffic = measured_traffic("attn_prefill_128k")
    attn_s = pre["attn_ms"] / 1e3
    # the memory side of the same kernel: the K/V rows every attended pair gathers (no reuse)
    # against the bytes that reached past L2 (FETCH_SIZE + WRITE_SIZE, copy-calibrated; these
    # include hits in the memory-side cache, so they bound the HBM bytes from above)
    memory_side = {"gathered_bytes_no_reuse": pre["gather_bytes"],
                   "io_bytes": pre["attn_bytes"] - pre["gather_bytes"],
                   "gathered_GBps": pre["gather_bytes"] / attn_s / 1e9,
                   "past_L2_bytes": traffic,
                   "past_L2_GBps": None if traffic is None else traffic / attn_s / 1e9,
                   "past_L2_frac_of_hbm_peak": (None if traffic is None else
                                                traffic / attn_s / 1e9 / PEAK_HBM_GBS),
                   "l2_reuse": None if traffic is None else pre["attn_bytes"] / traffic}
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "L": wl.L, "q_heads": s.num_q_heads,
                   "kv_heads": s.num_kv_heads, "head_dim": s.head_dim, "proxy_dim": s.proxy_dim,
                   "block_size": s.block_size, "topk_blocks": s.topk_blocks},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": "k_attn_prefill_resident<192>",
                     "launch": prefill_launches(wl),
                     "algorithmic_flops": pre["attn_flops"],
                     "flops_per_attended_pair": 4 * s.head_dim * s.num_q_heads,
                     "attended_pairs": pre["pairs"],
                     "memory_side": memory_side},
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "stages_ms": {"index_build": pre["build_ms"], "indexer_topk": pre["topk_ms"],
                      "sparse_attn_prefill": pre["attn_ms"]},
        "indexer_share": (pre["build_ms"] + pre["topk_ms"]) / pre["sequential_ms"],
        "schedule": (f"one stream: index build, then top-k and sparse attention over "
                     f"{PREFILL_CHUNKS} row range(s); stages_ms time the same three calls with "
                     f"an event between them ({pre['sequential_ms']:.2f} ms per step)"),
    }
    if peaks is not None:
        line["roofline"]["frac_of_measured_mfma"] = attn_tflops / peaks["mfma_bf16_tflops"]
        line["roofline"]["frac_of_gather_roofline"] = attn_tflops / peaks["gather_roofline_tflops"]
    line["ms_per_step_median"] = pre["median_ms"]
    line["attention_ms_median"] = pre["attn_ms_median"]
    line["index_build"] = pre["index_build"]
    if chunked is not None:
        line["chunked_prefill"] = chunked
    line["sliding_window_attention"] = pre["swa"]
    line["index_build_from_keys"] = pre["fused_index"]
    line["attention_backward"] = pre["backward"]
    if cov is not None:
        line["coverage"] = cov
    if dec is not None:
        line["decode"] = {"workload": "decode-1m-x16", "us_per_layer": dec["us_median"],
                          "us_indexer_topk": dec["us_topk"], "us_attention": dec["us_attn"],
                          "GBps": dec["gbs"], "hbm_frac": dec["gbs"] / PEAK_HBM_GBS,
                          "algorithmic_bytes": dec["bytes"],
                          "timing": ("median of the steps, 512 MiB read between steps; "
                                     "us_per_layer from steps timed at their ends only, the "
                                     "split from steps with an event between the two calls")}
        if "cpu_baseline" in dec:
            line["decode"]["cpu_baseline"] = dec["cpu_baseline"]
        if peaks is not None:
            line["decode"]["hbm_frac_of_measured_read"] = dec["gbs"] / peaks["hbm_read_GBps"]
        f8 = dec["fp8"]
        line["decode_fp8_storage"] = {"workload": "decode-1m-x16", "storage": "e4m3 rows + fp32 "
                                      "scale per row (index, K, V)",
                                      "us_per_layer": f8["us_median"],
                                      "us_indexer_topk": f8["us_topk"],
                                      "us_attention": f8["us_attn"], "GBps": f8["gbs"],
                                      "hbm_frac": f8["gbs"] / PEAK_HBM_GBS,
                                      "algorithmic_bytes": f8["bytes"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
