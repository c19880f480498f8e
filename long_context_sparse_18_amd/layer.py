"""One prefill pass of the sparse layer for a single sequence, on one stream.

Every step runs in the library (:mod:`long_context_sparse_18_amd.sgqa`); this module only
orders the calls: the index build, then, for each of ``chunks`` row ranges, the range's top-k
selection followed by its sparse attention.  Each call computes exactly what it computes when
the three stages run one after the other over all rows, so the results are the same bits for
any number of chunks.

The stages share one stream on purpose.  The sparse attention with a workspace is a persistent
launch of exactly the workgroups the GPU holds at once, whose waves wait (for a bounded time)
until most waves of their XCD have finished a history range; a kernel running beside it keeps
some of those workgroups from starting, and the waiting waves then run into their bound at
every range.  Selections queued on a side stream under the attention of the chunk before took
the 128K layer to a median of 128 ms and a mean of 160-200 ms (up to ~300 ms), against a steady
115.9 ms (one chunk) or 117.0 ms (eight chunks) on one stream.
"""
from __future__ import annotations

import torch

from . import sgqa
from .configs import LayerShape


def prefill_layer(shape: LayerShape, d: dict, q_start: int, L: int, scale: float, kb, idx, out,
                  lse, topk_workspace, attn_workspace, chunks: int = 1, stream=None):
    """Index build, top-k and sparse attention of the rows ``d["Q"]`` (positions ``q_start``
    onwards) over an ``L``-token cache; ``d`` holds kp, qp, Q, K, V, G as the library takes
    them.  Every call goes on ``stream`` (default: the current stream), the rows in ``chunks``
    consecutive ranges, each range's selection right before its attention."""
    stream = stream if stream is not None else torch.cuda.current_stream(d["Q"].device)
    T = d["Q"].shape[0]
    sgqa.index_build(shape, d["kp"], kb, [L], stream=stream)
    chunks = max(1, min(chunks, T))
    bounds = [T * c // chunks for c in range(chunks + 1)]
    for c in range(chunks):
        r0, r1 = bounds[c], bounds[c + 1]
        sgqa.indexer_topk(shape, d["qp"][r0:r1], kb, [q_start + r0], idx[r0:r1],
                          workspace=topk_workspace, stream=stream)
        sgqa.sparse_attn_prefill(shape, d["Q"][r0:r1], d["K"], d["V"], d["G"][r0:r1], idx[r0:r1],
                                 q_start + r0, L, scale, out[r0:r1],
                                 None if lse is None else lse[r0:r1], workspace=attn_workspace,
                                 stream=stream)
