"""Seeded synthetic inputs for the Sparse GQA layer (no arithmetic of the layer itself).

The pages publish no data for this path (ai.info "Sparse GQA targets
million-token context" quotes coverage from StepFun's own, unpublished
experiment), so every tensor here is synthetic:

* Q, V and the gate logits are i.i.d. N(0, 1).
* K follows an AR(1) process along the sequence, one independent stream per
  (sequence, KV head, dim): K_0 ~ N(0,1), K_t = rho*K_{t-1} + sqrt(1-rho^2)*e_t
  with rho = 0.9 (stationary variance 1).  Optionally the stream restarts from
  a fresh N(0,1) draw at every multiple of ``reseed_every``.
* Proxy keys: kp[t] = concat_g K[t, g, :] @ W_k, W_k ~ N(0,1)/sqrt(Hkv*d).
  Proxy queries: qp[t] = mean_h Q[t, h, :] @ W_q, W_q ~ N(0,1)/sqrt(d).
  The pages give only proxy_dim 256 (phantomic12 sparse_config); these
  projections stand in for the trained indexer weights.

The state is fp32 and every stored tensor is bf16.  Sub-streams are keyed
by (seed, tensor id, sequence) so that each tensor can be regenerated alone.
This module is shared by the tests, the benchmark and the smoke check; it
computes neither block representations, scores, selections nor attention.
"""
from __future__ import annotations

import math

import torch

from .configs import Workload

_TID = {"Q": 1, "K": 2, "V": 3, "G": 4, "Wq": 5, "Wk": 6}


def _gen(seed: int, tensor: str, seq: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TID[tensor] * 10_007 + seq * 101 + 12345) % (2**62))
    return g


def _randn_bf16(rows: int, cols: int, gen: torch.Generator, device, out=None,
                chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0,1) rows x cols, drawn in fp32 in row chunks and stored bf16."""
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    step = max(1, chunk_elems // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = torch.randn((r1 - r0, cols), generator=gen, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def ar1_stream(L: int, width: int, gen: torch.Generator, device, rho: float = 0.9,
               reseed_every: int | None = None) -> torch.Tensor:
    """fp32 [L, width] AR(1) along dim 0 with unit stationary variance.

    x_t = a_t * x_{t-1} + b_t * e_t with a_t = rho, b_t = sqrt(1 - rho^2), except
    a_t = 0, b_t = 1 at t = 0 and at every restart.  Evaluated as a log-depth
    doubling scan; the products a_t...a_{t-o} reach exactly 0 in fp32 after about
    ten doublings, which ends the scan.
    """
    x = torch.randn((L, width), generator=gen, device=device, dtype=torch.float32)
    a = torch.full((L,), rho, dtype=torch.float32, device=device)
    b = torch.full((L,), math.sqrt(1.0 - rho * rho), dtype=torch.float32, device=device)
    a[0] = 0.0
    b[0] = 1.0
    if reseed_every:
        a[::reseed_every] = 0.0
        b[::reseed_every] = 1.0
    x.mul_(b[:, None])
    off = 1
    while off < L:
        if not bool((a[off:] != 0).any()):
            break
        x[off:] = x[off:] + a[off:, None] * x[:-off]
        a[off:] = a[off:] * a[:-off]
        off *= 2
    return x


def proxy_weights(wl: Workload, seed: int, device):
    """(W_q [d, P], W_k [Hkv*d, P]) fp32, N(0,1) scaled by 1/sqrt(fan_in)."""
    s = wl.shape
    wq = torch.randn((s.head_dim, s.proxy_dim), generator=_gen(seed, "Wq", 0, device),
                     device=device, dtype=torch.float32) / math.sqrt(s.head_dim)
    fan = s.num_kv_heads * s.head_dim
    wk = torch.randn((fan, s.proxy_dim), generator=_gen(seed, "Wk", 0, device),
                     device=device, dtype=torch.float32) / math.sqrt(fan)
    return wq, wk


def _project_rows(x_bf16_2d: torch.Tensor, w: torch.Tensor, chunk: int = 1 << 16) -> torch.Tensor:
    out = torch.empty((x_bf16_2d.shape[0], w.shape[1]), dtype=torch.bfloat16,
                      device=x_bf16_2d.device)
    for r0 in range(0, x_bf16_2d.shape[0], chunk):
        r1 = min(x_bf16_2d.shape[0], r0 + chunk)
        out[r0:r1] = (x_bf16_2d[r0:r1].float() @ w).to(torch.bfloat16)
    return out


def make_cache(wl: Workload, seed: int, device, seq: int = 0, K_out=None, V_out=None,
               kp_out=None):
    """K, V [L, Hkv, d] bf16 and proxy keys kp [L, P] bf16 for one sequence."""
    s = wl.shape
    width = s.num_kv_heads * s.head_dim
    if K_out is None:
        K_out = torch.empty((wl.L, s.num_kv_heads, s.head_dim), dtype=torch.bfloat16,
                            device=device)
    if V_out is None:
        V_out = torch.empty_like(K_out)
    if kp_out is None:
        kp_out = torch.empty((wl.L, s.proxy_dim), dtype=torch.bfloat16, device=device)
    kf = ar1_stream(wl.L, width, _gen(seed, "K", seq, device), device, wl.rho, wl.reseed_every)
    K_out.view(wl.L, width).copy_(kf.to(torch.bfloat16))
    del kf
    _randn_bf16(wl.L, width, _gen(seed, "V", seq, device), device, out=V_out.view(wl.L, width))
    _, wk = proxy_weights(wl, seed, device)
    kp_out.copy_(_project_rows(K_out.view(wl.L, width), wk))
    return K_out, V_out, kp_out


def make_queries(wl: Workload, seed: int, device, seq: int = 0, T: int | None = None):
    """Q [T, Hq, d], gate logits G [T, Hq] and proxy queries qp [T, P], all bf16."""
    s = wl.shape
    T = wl.T if T is None else T
    Q = _randn_bf16(T, s.num_q_heads * s.head_dim, _gen(seed, "Q", seq, device), device)
    Q = Q.view(T, s.num_q_heads, s.head_dim)
    G = _randn_bf16(T, s.num_q_heads, _gen(seed, "G", seq, device), device)
    wq, _ = proxy_weights(wl, seed, device)
    qp = torch.empty((T, s.proxy_dim), dtype=torch.bfloat16, device=device)
    chunk = 1 << 14
    for r0 in range(0, T, chunk):
        r1 = min(T, r0 + chunk)
        qp[r0:r1] = (Q[r0:r1].float().mean(dim=1) @ wq).to(torch.bfloat16)
    return Q, G, qp


def make_prefill(wl: Workload, seed: int, device):
    """All tensors of a single-sequence prefill workload."""
    K, V, kp = make_cache(wl, seed, device)
    Q, G, qp = make_queries(wl, seed, device)
    return dict(Q=Q, K=K, V=V, G=G, kp=kp, qp=qp)


def make_decode(wl: Workload, seed: int, device, nseq: int | None = None):
    """Batched decode inputs: caches [nseq, L, Hkv, d], kp [nseq, L, P] and one query each."""
    s = wl.shape
    nseq = wl.nseq if nseq is None else nseq
    K = torch.empty((nseq, wl.L, s.num_kv_heads, s.head_dim), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    kp = torch.empty((nseq, wl.L, s.proxy_dim), dtype=torch.bfloat16, device=device)
    Q = torch.empty((nseq, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=device)
    G = torch.empty((nseq, s.num_q_heads), dtype=torch.bfloat16, device=device)
    qp = torch.empty((nseq, s.proxy_dim), dtype=torch.bfloat16, device=device)
    for b in range(nseq):
        make_cache(wl, seed, device, seq=b, K_out=K[b], V_out=V[b], kp_out=kp[b])
        q, g, p = make_queries(wl, seed, device, seq=b, T=1)
        Q[b].copy_(q[0])
        G[b].copy_(g[0])
        qp[b].copy_(p[0])
    return dict(Q=Q, K=K, V=V, G=G, kp=kp, qp=qp)


def bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor as a host numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
