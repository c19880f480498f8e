"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` takes a loaded oracle library (the real one, or a copy with a
planted mistake) and raises ``AssertionError`` when the oracle disagrees with
something it does not itself define: a closed form, a textbook or library
routine on a special case, an invariant, or a brute-force count.  None of them
re-types the oracle's own formula.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def bf16_bits(x) -> np.ndarray:
    """float array -> raw bf16 bits (round to nearest even, via torch)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    """raw bf16 bits -> float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def small_problem(L=96, Hq=8, Hkv=2, d=64, P=32, seed=0):
    rng = np.random.default_rng(seed)
    return dict(
        Q=bf16_bits(rng.standard_normal((L, Hq, d))),
        K=bf16_bits(rng.standard_normal((L, Hkv, d))),
        V=bf16_bits(rng.standard_normal((L, Hkv, d))),
        G=bf16_bits(rng.standard_normal((L, Hq))),
        kp=bf16_bits(rng.standard_normal((L, P))),
        qp=bf16_bits(rng.standard_normal((L, P))),
    )


def lexsort_selection(scores_row: np.ndarray, c: int, k: int) -> np.ndarray:
    """Textbook selection: numpy lexsort by (score desc, index asc), own block added."""
    if c <= k - 1:
        sel = np.arange(c + 1)
    else:
        s = scores_row[:c]
        order = np.lexsort((np.arange(c), -s))
        sel = np.sort(np.concatenate([order[: k - 1], [c]]))
    out = np.full(k, -1, dtype=np.int32)
    out[: len(sel)] = sel
    return out


def sdpa_reference(p, mask: np.ndarray, scale: float):
    """Library attention: torch SDPA in fp64 with KV heads repeated, times sigmoid(gate)."""
    Q = torch.from_numpy(widen(p["Q"]))  # [T, Hq, d]
    K = torch.from_numpy(widen(p["K"]))
    V = torch.from_numpy(widen(p["V"]))
    G = torch.from_numpy(widen(p["G"]))
    Hq, Hkv = Q.shape[1], K.shape[1]
    rep = Hq // Hkv
    q = Q.permute(1, 0, 2)
    k = K.permute(1, 0, 2).repeat_interleave(rep, dim=0)
    v = V.permute(1, 0, 2).repeat_interleave(rep, dim=0)
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    o = o.permute(1, 0, 2) * torch.sigmoid(G)[:, :, None]
    return o.numpy()


def oracle_full_layer(lib, p, B, k, scale):
    """Oracle steps 1-4 for every row of a small single-sequence prefill."""
    L = p["K"].shape[0]
    t = np.arange(L, dtype=np.int64)
    kb = oracle.index_build(p["kp"], B, lib=lib)
    width = max(1, (L - 1) // B)
    sc = oracle.scores(p["qp"], t, B, kb, width=width, lib=lib)
    idx = oracle.topk(sc, t, B, k, lib=lib)
    out, lse = oracle.sparse_attention(p["Q"], t, p["K"], p["V"], p["G"], idx, B, scale, lib=lib)
    return kb, sc, idx, out, lse


# --------------------------------------------------------------------------- index
def pin_index_b1_identity(lib):
    """B = 1: every block is one token, so its mean is the token's proxy key, bit for bit."""
    p = small_problem()
    kb = oracle.index_build(p["kp"], 1, lib=lib)
    assert np.array_equal(kb, widen(p["kp"]))


def pin_index_closed_form(lib):
    """kp[s][p] = s + p (exact in bf16 for s+p < 256): block j's mean is first + (n-1)/2 + p,
    with n = 8 for full blocks and n = 3 for the trailing block of L = 43."""
    L, P, B = 43, 16, 8
    vals = np.arange(L)[:, None] + np.arange(P)[None, :]
    kb = oracle.index_build(bf16_bits(vals), B, lib=lib)
    assert kb.shape == (6, P)
    for j in range(6):
        n = min(B, L - j * B)
        want = j * B + (n - 1) / 2.0 + np.arange(P)
        assert np.array_equal(kb[j], want), (j, kb[j], want)


def pin_index_from_keys_project_then_average(lib):
    """Linearity: projecting each block's mean key equals averaging the projected keys,
    computed the other way round with a numpy fp64 matmul, trailing partial block included
    (L = 43, B = 8: five full blocks and one of 3 tokens)."""
    rng = np.random.default_rng(21)
    L, Hkv, d, P, B = 43, 2, 24, 16, 8
    K = bf16_bits(rng.standard_normal((L, Hkv, d)))
    wt = bf16_bits(rng.standard_normal((P, Hkv * d)) / math.sqrt(Hkv * d))
    kb = oracle.index_build_from_keys(K, wt, B, lib=lib)
    kp = widen(K).reshape(L, -1) @ widen(wt).T  # [L, P]
    want = np.stack([kp[j * B: min(L, (j + 1) * B)].mean(axis=0) for j in range(-(-L // B))])
    assert kb.shape == want.shape
    assert np.allclose(kb, want, rtol=1e-12, atol=1e-12), np.abs(kb - want).max()
    kb1 = oracle.index_build_from_keys(K, wt, 1, lib=lib)
    assert np.allclose(kb1, kp, rtol=1e-12, atol=1e-12)


def pin_index_from_keys_selection_matrix(lib):
    """W = a coordinate selection (rows of the identity, permuted): the fused build must equal
    the proxy-key block compression of the selected key coordinates, bit for bit."""
    rng = np.random.default_rng(22)
    L, Hkv, d, B = 61, 2, 16, 8
    width = Hkv * d
    K = bf16_bits(rng.standard_normal((L, Hkv, d)))
    pick = rng.permutation(width)[:12]
    wt = np.zeros((len(pick), width))
    wt[np.arange(len(pick)), pick] = 1.0
    kb = oracle.index_build_from_keys(K, bf16_bits(wt), B, lib=lib)
    kp = K.reshape(L, width)[:, pick]
    assert np.array_equal(kb, oracle.index_build(np.ascontiguousarray(kp), B, lib=lib))


# --------------------------------------------------------------------------- scores
def pin_scores_basis(lib):
    """qp = unit vector e_p picks column p of kb; only blocks j < floor(t/B) are scored."""
    P, B = 32, 8
    rng = np.random.default_rng(3)
    kb = rng.standard_normal((40, P))
    t = np.array([0, 7, 8, 15, 16, 100, 319], dtype=np.int64)
    cols = np.array([0, 5, 31, 2, 17, 9, 30])
    qp = np.zeros((len(t), P))
    qp[np.arange(len(t)), cols] = 1.0
    sc = oracle.scores(bf16_bits(qp), t, B, kb, width=40, lib=lib)
    for r, (tt, cc) in enumerate(zip(t, cols)):
        c = tt // B
        assert np.array_equal(sc[r, :c], kb[:c, cc]), (tt, cc)
        assert np.all(np.isnan(sc[r, c:])), (tt, "scored a block that is not a complete past block")


def pin_scores_bilinear(lib):
    """score(a*qp1 + b*qp2) = a*score(qp1) + b*score(qp2) with exactly representable weights,
    and swapping the roles of P coordinates permutes nothing (sum is symmetric)."""
    P, B = 32, 8
    rng = np.random.default_rng(5)
    kb = rng.standard_normal((20, P))
    q1 = bf16_bits(rng.integers(-4, 5, size=(1, P)).astype(np.float64))
    q2 = bf16_bits(rng.integers(-4, 5, size=(1, P)).astype(np.float64))
    q3 = bf16_bits(2.0 * widen(q1) - widen(q2))
    t = np.array([160], dtype=np.int64)
    s1 = oracle.scores(q1, t, B, kb, width=20, lib=lib)
    s2 = oracle.scores(q2, t, B, kb, width=20, lib=lib)
    s3 = oracle.scores(q3, t, B, kb, width=20, lib=lib)
    np.testing.assert_allclose(s3, 2 * s1 - s2, rtol=0, atol=1e-12)
    perm = rng.permutation(P)
    s4 = oracle.scores(np.ascontiguousarray(q1[:, perm]), t, B, np.ascontiguousarray(kb[:, perm]),
                       width=20, lib=lib)
    np.testing.assert_allclose(s4, s1, rtol=0, atol=1e-12)
    # a non-symmetric kb probe: reversing P on the query alone must change the scores
    s5 = oracle.scores(np.ascontiguousarray(q1[:, ::-1]), t, B, kb, width=20, lib=lib)
    dense = widen(q1)[0][::-1] @ kb.T
    np.testing.assert_allclose(s5[0], dense, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- top-k
def pin_topk_lexsort(lib):
    """Against numpy.lexsort on rows full of exact ties (scores drawn from 5 values)."""
    B, k = 8, 6
    rng = np.random.default_rng(7)
    t = np.arange(0, 400, 3, dtype=np.int64)
    width = 400 // B
    sc = rng.integers(0, 5, size=(len(t), width)).astype(np.float64)
    idx = oracle.topk(sc, t, B, k, lib=lib)
    for r, tt in enumerate(t):
        want = lexsort_selection(sc[r], int(tt // B), k)
        assert np.array_equal(idx[r], want), (tt, idx[r], want)


def pin_topk_invariants(lib):
    """Causal, own block kept, |S| = min(k, c+1), ascending, unique, -1 padding at the end."""
    rng = np.random.default_rng(11)
    for B, k in ((8, 4), (8, 16), (1, 8), (1, 1), (8, 1)):
        t = rng.integers(0, 2000, size=60).astype(np.int64)
        width = int(t.max()) // B + 1
        sc = rng.standard_normal((len(t), width))
        idx = oracle.topk(sc, t, B, k, lib=lib)
        for r, tt in enumerate(t):
            c = int(tt // B)
            row = idx[r]
            valid = row[row >= 0]
            assert len(valid) == min(k, c + 1)
            assert np.all(row[len(valid):] == -1)
            assert np.all(np.diff(valid) > 0)
            assert valid[-1] == c
            assert valid.max() <= c


def pin_topk_planted(lib):
    """End to end through index, scores and top-k: blocks whose proxy keys all equal +u
    (u = the query's proxy) must be exactly the selection; the rest have kp = -u."""
    B, k, P = 8, 5, 32
    nblk = 30
    L = nblk * B
    rng = np.random.default_rng(13)
    u = np.sign(rng.standard_normal(P))
    planted = np.sort(rng.choice(nblk - 1, size=k - 1, replace=False))
    kp = np.tile(-u, (L, 1))
    for j in planted:
        kp[j * B:(j + 1) * B] = u
    kbits = bf16_bits(kp)
    t = np.array([L - 1], dtype=np.int64)
    kb = oracle.index_build(kbits, B, lib=lib)
    sc = oracle.scores(bf16_bits(u[None, :]), t, B, kb, width=nblk, lib=lib)
    idx = oracle.topk(sc, t, B, k, lib=lib)
    want = np.sort(np.concatenate([planted, [nblk - 1]]))
    assert np.array_equal(idx[0], want), (idx[0], want)


# --------------------------------------------------------------------------- attention
def _mask_from_selection(idx: np.ndarray, B: int, L: int) -> np.ndarray:
    """Boolean [T, L] mask built directly from selected block ids (not from the oracle)."""
    T = idx.shape[0]
    blk = np.arange(L) // B
    m = np.zeros((T, L), dtype=bool)
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        m[t] = np.isin(blk, sel) & (np.arange(L) <= t)
    return m


def pin_attention_dense_sdpa(lib):
    """k covers every block: sparse attention is dense causal GQA (torch SDPA, fp64)."""
    p = small_problem()
    L = p["K"].shape[0]
    d = p["Q"].shape[2]
    scale = 1.0 / math.sqrt(d)
    for B in (8, 1):
        k = L // B + 1
        _, _, idx, out, _ = oracle_full_layer(lib, p, B, k, scale)
        ref = sdpa_reference(p, np.tril(np.ones((L, L), dtype=bool)), scale)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_attention_sparse_sdpa(lib):
    """Any selection: equal to SDPA under the block mask built from the selected ids."""
    p = small_problem(seed=1)
    L = p["K"].shape[0]
    d = p["Q"].shape[2]
    scale = 1.0 / math.sqrt(d)
    for B, k in ((8, 4), (8, 1), (1, 5), (8, 2)):
        _, sc, idx, out, _ = oracle_full_layer(lib, p, B, k, scale)
        ref = sdpa_reference(p, _mask_from_selection(idx, B, L), scale)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_attention_t0_closed_form(lib):
    """At t = 0 the only token is itself: out[0, h] = sigmoid(G[0, h]) * V[0, g(h)]."""
    p = small_problem(seed=2)
    d = p["Q"].shape[2]
    _, _, _, out, lse = oracle_full_layer(lib, p, 8, 4, 1.0 / math.sqrt(d))
    V0 = widen(p["V"])[0]
    G0 = widen(p["G"])[0]
    Hq, Hkv = p["Q"].shape[1], p["K"].shape[1]
    for h in range(Hq):
        g = h // (Hq // Hkv)
        np.testing.assert_allclose(out[0, h], V0[g] / (1.0 + np.exp(-G0[h])), rtol=0, atol=1e-15)
        # one token: lse is its logit
        z = (widen(p["Q"])[0, h] @ widen(p["K"])[0, g]) / math.sqrt(d)
        np.testing.assert_allclose(lse[0, h], z, rtol=0, atol=1e-12)


def pin_attention_constant_keys(lib):
    """All keys equal: every logit is the same z0, so lse = z0 + ln|U_t| and the output is
    sigmoid(G) times the plain mean of V over the attended tokens."""
    p = small_problem(seed=4)
    L, Hkv, d = p["K"].shape
    Hq = p["Q"].shape[1]
    K = np.broadcast_to(p["K"][:1], p["K"].shape).copy()
    p = dict(p, K=K)
    B, k = 8, 3
    scale = 1.0 / math.sqrt(d)
    _, _, idx, out, lse = oracle_full_layer(lib, p, B, k, scale)
    Vw, Qw, Kw, Gw = widen(p["V"]), widen(p["Q"]), widen(K), widen(p["G"])
    blk = np.arange(L) // B
    for t in (0, 5, 8, 23, 40, 95):
        sel = idx[t][idx[t] >= 0]
        toks = np.nonzero(np.isin(blk, sel) & (np.arange(L) <= t))[0]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            z0 = scale * (Qw[t, h] @ Kw[0, g])
            np.testing.assert_allclose(lse[t, h], z0 + math.log(len(toks)), rtol=0, atol=1e-12)
            want = Vw[toks, g].mean(axis=0) / (1.0 + math.exp(-Gw[t, h]))
            np.testing.assert_allclose(out[t, h], want, rtol=0, atol=1e-12)


def pin_attention_bounds(lib):
    """Convexity: sigmoid(G)*min_U V <= out <= sigmoid(G)*max_U V, per dimension."""
    p = small_problem(seed=6)
    L, Hkv, d = p["K"].shape
    Hq = p["Q"].shape[1]
    B, k = 8, 3
    _, _, idx, out, _ = oracle_full_layer(lib, p, B, k, 1.0 / math.sqrt(d))
    Vw, Gw = widen(p["V"]), widen(p["G"])
    blk = np.arange(L) // B
    for t in range(L):
        sel = idx[t][idx[t] >= 0]
        toks = np.nonzero(np.isin(blk, sel) & (np.arange(L) <= t))[0]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            sg = 1.0 / (1.0 + math.exp(-Gw[t, h]))
            lo = sg * Vw[toks, g].min(axis=0) - 1e-12
            hi = sg * Vw[toks, g].max(axis=0) + 1e-12
            assert np.all(out[t, h] >= lo) and np.all(out[t, h] <= hi), (t, h)


def pin_coverage_identity(lib):
    """exp(lse_sparse - lse_dense) is the dense softmax mass on the selected tokens
    (library softmax over the masked fp64 logits)."""
    p = small_problem(seed=8)
    L, Hkv, d = p["K"].shape
    Hq = p["Q"].shape[1]
    scale = 1.0 / math.sqrt(d)
    B = 8
    _, _, idx_s, _, lse_s = oracle_full_layer(lib, p, B, 3, scale)
    _, _, _, _, lse_d = oracle_full_layer(lib, p, B, L // B + 1, scale)
    Q = torch.from_numpy(widen(p["Q"]))
    K = torch.from_numpy(widen(p["K"]))
    logits = torch.einsum("thd,sgd->thgs", Q, K)  # all (head, group) pairs
    mask = _mask_from_selection(idx_s, B, L)
    causal = np.tril(np.ones((L, L), dtype=bool))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        z = logits[:, h, g, :] * scale
        z = z.masked_fill(~torch.from_numpy(causal), float("-inf"))
        w = torch.softmax(z, dim=-1).numpy()
        mass = (w * mask).sum(axis=1)
        np.testing.assert_allclose(np.exp(lse_s[:, h] - lse_d[:, h]), mass, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- sliding window
def pin_window_dense_and_band(lib):
    """Window covering the whole prefix is dense causal attention; any window equals SDPA
    under the band mask t-W < s <= t (torch, fp64)."""
    p = small_problem(seed=9)
    L, Hkv, d = p["K"].shape
    scale = 1.0 / math.sqrt(d)
    t = np.arange(L, dtype=np.int64)
    for W in (L, 1000, 17, 8, 2):
        out, _ = oracle.window_attention(p["Q"], t, p["K"], p["V"], p["G"], W, scale, lib=lib)
        s_ = np.arange(L)
        band = (s_[None, :] <= t[:, None]) & (s_[None, :] > t[:, None] - W)
        np.testing.assert_allclose(out, sdpa_reference(p, band, scale), rtol=0, atol=1e-12)


def pin_window_one_closed_form(lib):
    """W = 1: each query sees only itself, out = sigmoid(G) V[t] and lse = its own logit."""
    p = small_problem(seed=10)
    L, Hkv, d = p["K"].shape
    Hq = p["Q"].shape[1]
    t = np.arange(L, dtype=np.int64)
    out, lse = oracle.window_attention(p["Q"], t, p["K"], p["V"], p["G"], 1, 1.0 / math.sqrt(d),
                                       lib=lib)
    Qw, Kw, Vw, Gw = widen(p["Q"]), widen(p["K"]), widen(p["V"]), widen(p["G"])
    for h in range(Hq):
        g = h // (Hq // Hkv)
        np.testing.assert_allclose(out[:, h], Vw[:, g] / (1 + np.exp(-Gw[:, h]))[:, None],
                                   rtol=0, atol=1e-15)
        z = np.einsum("td,td->t", Qw[:, h], Kw[:, g]) / math.sqrt(d)
        np.testing.assert_allclose(lse[:, h], z, rtol=0, atol=1e-12)


def pin_window_token_count(lib):
    """The window holds min(W, t+1) positions ending at t."""
    for t_, W in ((0, 512), (5, 512), (511, 512), (512, 512), (100000, 512), (7, 1)):
        toks = np.empty(max(1, W), dtype=np.int64)
        n = lib.orc_window_token_set(t_, W, oracle._ptr(toks))
        assert n == min(W, t_ + 1)
        assert toks[n - 1] == t_ and toks[0] == t_ - n + 1


# --------------------------------------------------------------------------- backward
def _autograd_reference(p, mask: np.ndarray, scale: float, gout: np.ndarray):
    """Library gradients: torch autograd through fp64 SDPA (KV heads repeated, block mask)
    times sigmoid(gate), for the loss sum(out * gout)."""
    Q = torch.from_numpy(widen(p["Q"])).requires_grad_(True)
    K = torch.from_numpy(widen(p["K"])).requires_grad_(True)
    V = torch.from_numpy(widen(p["V"])).requires_grad_(True)
    G = torch.from_numpy(widen(p["G"])).requires_grad_(True)
    rep = Q.shape[1] // K.shape[1]
    q = Q.permute(1, 0, 2)
    k = K.permute(1, 0, 2).repeat_interleave(rep, dim=0)
    v = V.permute(1, 0, 2).repeat_interleave(rep, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask),
                                                         scale=scale)
    out = o.permute(1, 0, 2) * torch.sigmoid(G)[:, :, None]
    (out * torch.from_numpy(gout)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy(), G.grad.numpy()


def pin_backward_autograd(lib):
    """The fixed-selection backward equals torch autograd through SDPA (fp64) under the mask
    built from the selected blocks, for a sparse (k = 4) and a dense selection; and the sums
    over key rows obey sum_s dV[s][g] = sum_t sum_{h in g} sigmoid(G) gout and
    sum_s dK[s][g] = 0 (the dz of each (t, h) sum to zero)."""
    p = small_problem(seed=12)
    L, Hkv, d = p["K"].shape
    Hq = p["Q"].shape[1]
    rng = np.random.default_rng(13)
    gout = bf16_bits(rng.standard_normal((L, Hq, d)))
    scale = 1 / math.sqrt(d)
    t = np.arange(L, dtype=np.int64)
    for B, k in ((8, 4), (8, 64)):
        kb = oracle.index_build(p["kp"], B, lib=lib)
        sc = oracle.scores(p["qp"], t, B, kb, width=max(1, (L - 1) // B), lib=lib)
        idx = oracle.topk(sc, t, B, k, lib=lib)
        mask = np.zeros((L, L), dtype=bool)
        for r in range(L):
            mask[r, oracle.token_set(idx[r], B, r, lib=lib)] = True
        dq, dK, dV, dg = oracle.sparse_attention_backward(p["Q"], t, p["K"], p["V"], p["G"], idx,
                                                          B, scale, gout, lib=lib)
        rq, rK, rV, rg = _autograd_reference(p, mask, scale, widen(gout))
        for ours, ref in ((dq, rq), (dK, rK), (dV, rV), (dg, rg)):
            assert np.allclose(ours, ref, rtol=1e-9, atol=1e-11), np.abs(ours - ref).max()
        sg = 1 / (1 + np.exp(-widen(p["G"])))
        want_v = (sg[:, :, None] * widen(gout)).reshape(L, Hkv, Hq // Hkv, d).sum(axis=(0, 2))
        assert np.allclose(dV.sum(axis=0), want_v, rtol=1e-10, atol=1e-10)
        assert np.allclose(dK.sum(axis=0), 0.0, atol=1e-10)


# --------------------------------------------------------------------------- FP8 storage
def _torch_e4m3_bits(values) -> np.ndarray:
    """Library cast: torch float32 -> float8_e4m3fn (round to nearest even), as codes."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_library(lib):
    """All 256 E4M3 codes decode to torch's float8_e4m3fn values (NaN codes to NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes, lib=lib)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def pin_e4m3_encode_library(lib):
    """Encoding equals torch's round-to-nearest-even cast on every representable value, every
    midpoint, one float32 ulp either side of each midpoint, and random values in range;
    magnitudes from 448 up saturate to the largest finite code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = np.unique(vals[~np.isnan(vals)])
    mids = (vals[1:] + vals[:-1]) / 2
    mids = mids.astype(np.float32)
    probe = np.concatenate([vals.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                            np.nextafter(mids, np.float32(-np.inf)),
                            np.random.default_rng(31).uniform(-448, 448, 4000).astype(np.float32),
                            np.random.default_rng(32).uniform(-0.02, 0.02, 4000).astype(np.float32)])
    probe = probe[np.abs(probe) <= 448]
    assert np.array_equal(oracle.e4m3_encode(probe, lib=lib), _torch_e4m3_bits(probe))
    sat = np.array([448.0, 460.0, 500.0, 1e6, -448.0, -1e6], dtype=np.float32)
    assert oracle.e4m3_encode(sat, lib=lib).tolist() == [0x7E] * 4 + [0xFE] * 2


def pin_quantize_rows_error_bound(lib):
    """Row quantisation: the dequantised value is within half an E4M3 spacing (times the row
    scale) of the input, the row's largest magnitude lands on a code of magnitude >= 416 (the
    top two E4M3 values), and a zero row gives zero codes."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((50, 192)) * np.exp(rng.uniform(-6, 6, (50, 1)))
    x[7] = 0.0
    bits = bf16_bits(x)
    codes, scales = oracle.quantize_rows(bits, lib=lib)
    deq = oracle.dequant_rows(codes, scales, lib=lib)
    xv = widen(bits)
    y = np.abs(xv) / scales[:, None].astype(np.float64)
    spacing = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 3))
    assert np.all(np.abs(deq - xv) <= 0.5 * spacing * scales[:, None] * (1 + 1e-6))
    top = np.abs(oracle.e4m3_decode(codes, lib=lib)).max(axis=1)
    assert np.all(top[np.arange(50) != 7] >= 416) and np.all(top <= 448)
    assert np.all(codes[7] == 0)


def pin_attend_f64_sdpa(lib):
    """The attention core on float64 rows (dequantised FP8) equals torch SDPA in fp64, and on
    widened bf16 rows it equals the bf16 entry bit for bit."""
    rng = np.random.default_rng(34)
    n, Hq, Hkv, d = 37, 8, 2, 64
    q = bf16_bits(rng.standard_normal((Hq, d)))
    g = bf16_bits(rng.standard_normal(Hq))
    K = rng.standard_normal((n, Hkv, d)) * 0.7
    V = rng.standard_normal((n, Hkv, d))
    scale = 1 / math.sqrt(d)
    out, lse = oracle.attend_f64(q, K, V, g, scale, lib=lib)
    Qt = torch.from_numpy(widen(q))[:, None, :]                       # [Hq, 1, d]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, scale=scale)[:, 0, :]
    o = o * torch.sigmoid(torch.from_numpy(widen(g)))[:, None]
    assert np.allclose(out, o.numpy(), rtol=1e-12, atol=1e-12)
    z = (torch.from_numpy(widen(q))[:, None, :] * Kt).sum(-1) * scale
    assert np.allclose(lse, torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12, atol=1e-12)
    kb, vb = bf16_bits(K), bf16_bits(V)
    o1, l1 = oracle.attend(q, kb, vb, g, scale, lib=lib)
    o2, l2 = oracle.attend_f64(q, widen(kb), widen(vb), g, scale, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


ALL_PINS = [
    pin_backward_autograd,
    pin_e4m3_decode_library,
    pin_e4m3_encode_library,
    pin_quantize_rows_error_bound,
    pin_attend_f64_sdpa,
    pin_index_b1_identity,
    pin_index_closed_form,
    pin_index_from_keys_project_then_average,
    pin_index_from_keys_selection_matrix,
    pin_scores_basis,
    pin_scores_bilinear,
    pin_topk_lexsort,
    pin_topk_invariants,
    pin_topk_planted,
    pin_attention_dense_sdpa,
    pin_attention_sparse_sdpa,
    pin_attention_t0_closed_form,
    pin_attention_constant_keys,
    pin_attention_bounds,
    pin_coverage_identity,
    pin_window_dense_and_band,
    pin_window_one_closed_form,
    pin_window_token_count,
]
