"""One prefill pass of the sparse layer for a single sequence, scheduled over two streams.

Every step runs in the library (:mod:`long_context_sparse_18_amd.sgqa`); this module only
orders the calls.  The index is built first; the query rows are then cut into ``chunks`` row
ranges, the top-k selections of all ranges are queued on a side stream, and the attention of
range i waits only for range i's selection.  The selection of the next ranges therefore runs
under the attention of the current one.  Each call computes exactly what it computes when the
three stages run one after the other, so the results are the same bits.
"""
from __future__ import annotations

import torch

from . import sgqa
from .configs import LayerShape


def prefill_layer(shape: LayerShape, d: dict, q_start: int, L: int, scale: float, kb, idx, out,
                  lse, topk_workspace, attn_workspace, chunks: int = 8, stream=None,
                  side_stream=None):
    """Index build, top-k and sparse attention of the rows ``d["Q"]`` (positions ``q_start``
    onwards) over an ``L``-token cache; ``d`` holds kp, qp, Q, K, V, G as the library takes
    them.  ``stream`` (default: the current stream) carries the index build and the attention,
    ``side_stream`` (required) the selections; on return ``stream`` has waited for all of it."""
    if side_stream is None:
        raise ValueError("prefill_layer needs a side stream for the selections")
    stream = stream if stream is not None else torch.cuda.current_stream(d["Q"].device)
    T = d["Q"].shape[0]
    sgqa.index_build(shape, d["kp"], kb, [L], stream=stream)
    built = torch.cuda.Event()
    built.record(stream)
    side_stream.wait_event(built)
    chunks = max(1, min(chunks, T))
    bounds = [T * c // chunks for c in range(chunks + 1)]
    ready = []
    for c in range(chunks):
        r0, r1 = bounds[c], bounds[c + 1]
        sgqa.indexer_topk(shape, d["qp"][r0:r1], kb, [q_start + r0], idx[r0:r1],
                          workspace=topk_workspace, stream=side_stream)
        ev = torch.cuda.Event()
        ev.record(side_stream)
        ready.append(ev)
    for c in range(chunks):
        r0, r1 = bounds[c], bounds[c + 1]
        stream.wait_event(ready[c])
        sgqa.sparse_attn_prefill(shape, d["Q"][r0:r1], d["K"], d["V"], d["G"][r0:r1], idx[r0:r1],
                                 q_start + r0, L, scale, out[r0:r1],
                                 None if lse is None else lse[r0:r1], workspace=attn_workspace,
                                 stream=stream)
