"""The five synthetic workloads of the Sparse GQA layer, by shape.

Layer shape (phantomic12 "Step 5 Preview" catalogue entry, config.json part):
64 query heads, 4 attention groups (so 4 KV heads), head_dim 192, and
(sparse_config) topk 512 blocks with proxy_dim 256; block size 8 from ai.info
"Sparse GQA targets million-token context".  The tiny shape is a scaled-down
copy that a CPU finishes in seconds.

``q_start`` is the position of the first query token; queries occupy
``[q_start, q_start + T)`` and the cache holds ``L`` tokens.  The chunked
prefill workload keeps T = 8192 new tokens and L = 1 048 580 total tokens, so
the chunk starts at position 1 040 388 (offset 4 inside block 130 048).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class LayerShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    proxy_dim: int
    block_size: int
    topk_blocks: int

    @property
    def heads_per_group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    nseq: int
    T: int            # query tokens per sequence
    L: int            # cache tokens per sequence (after the queries are appended)
    q_start: int      # position of the first query token
    reseed_every: int | None = None   # key AR(1) stream restarts every this many tokens
    rho: float = 0.9

    @property
    def nblk(self) -> int:
        return -(-self.L // self.shape.block_size)


TINY = LayerShape(8, 2, 64, 32, 8, 16)
REAL = LayerShape(64, 4, 192, 256, 8, 512)

WORKLOADS = {
    0: Workload("tiny-1k", TINY, nseq=1, T=1024, L=1024, q_start=0),
    1: Workload("prefill-32k", REAL, nseq=1, T=32768, L=32768, q_start=0),
    2: Workload("prefill-128k", REAL, nseq=1, T=131072, L=131072, q_start=0),
    3: Workload("decode-1m-x16", REAL, nseq=16, T=1, L=1048576, q_start=1048575),
    4: Workload("chunked-prefill-1m", REAL, nseq=1, T=8192, L=1048580, q_start=1040388,
                reseed_every=65536),
}


def with_selection(shape: LayerShape, block_size: int, topk_blocks: int) -> LayerShape:
    """The same layer widths with another (block size, top-k) pair, e.g. B=1, k=2048."""
    return dataclasses.replace(shape, block_size=block_size, topk_blocks=topk_blocks)
