"""Checks that pin the fp64 oracle to facts fixed by the pages and by mathematics.

Each check takes `attn(q, k, v, causal, scale) -> (o, lse)` over fp64 numpy
arrays of shape (B, H, S, D) and raises AssertionError when the fact fails.
They run against the real oracle (tests/test_oracle.py) and against mutated
copies of it (tests/test_oracle_mutants.py), where every plausible mistake
must trip at least one of them.

None of them re-types the oracle's formula: each compares against something
else -- a streaming (online-softmax) evaluation, a closed form, an invariant,
a brute-force sum with math.fsum, or a library routine.
"""
from __future__ import annotations

import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# online softmax (infra.bea.ai guide, "Optimization 2: Delay Rescaling";
# cookbook Triton kernel loop) evaluated tile by tile in fp64
# ---------------------------------------------------------------------------
def online_softmax_attention(q, k, v, causal, scale, tile):
    """Streaming evaluation: running max m, running sum l and an unnormalised
    accumulator rescaled by exp(m_old - m_new) per key tile; divide by l once
    at the end. Written independently of the two-pass oracle."""
    B, H, S, D = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            s_full = scale * (q[b, h] @ k[b, h].T)  # (S, S)
            m = np.full(S, -np.inf)
            l = np.zeros(S)
            acc = np.zeros((S, D))
            for start in range(0, S, tile):
                cols = np.arange(start, min(start + tile, S))
                s = s_full[:, cols].copy()
                if causal:
                    s[np.arange(S)[:, None] < cols[None, :]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                # rows whose keys are all masked so far keep m = -inf
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                p = np.exp(s - ref[:, None])
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ v[b, h][cols]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse


def check_online_equals_two_pass(attn):
    rng = _rng(11)
    for causal in (False, True):
        for S in (1, 5, 13):
            q, k, v = (_randn(rng, (1, 2, S, 4)) for _ in range(3))
            o, lse = attn(q, k, v, causal, 0.7)
            for tile in sorted({1, 3, 7, S}):
                o2, lse2 = online_softmax_attention(q, k, v, causal, 0.7, tile)
                np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def check_v_ones_gives_ones(attn):
    rng = _rng(12)
    q, k = _randn(rng, (2, 2, 9, 8)), _randn(rng, (2, 2, 9, 8))
    v = np.ones((2, 2, 9, 8))
    for causal in (False, True):
        o, _ = attn(q, k, v, causal, 0.5)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)


def check_rows_sum_to_one(attn):
    """With S = D and V = I, O equals the probability matrix P itself."""
    rng = _rng(13)
    S = 6
    q, k = _randn(rng, (1, 1, S, S)), _randn(rng, (1, 1, S, S))
    v = np.eye(S)[None, None]
    for causal in (False, True):
        p, _ = attn(q, k, v, causal, 0.9)
        p = p[0, 0]
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert np.all(p[np.triu_indices(S, 1)] == 0.0)
        # the probabilities are ordered like the scores in every row
        s = (q[0, 0] @ k[0, 0].T)
        for i in range(S):
            n = i + 1 if causal else S
            assert np.array_equal(np.argsort(s[i, :n], kind="stable"),
                                  np.argsort(p[i, :n], kind="stable"))


def check_causal_row0(attn):
    """Causal row 0 sees only key 0: o_0 = v_0 exactly, lse_0 = scale q_0.k_0."""
    rng = _rng(14)
    q, k, v = (_randn(rng, (1, 3, 7, 5)) for _ in range(3))
    o, lse = attn(q, k, v, True, 0.3)
    for h in range(3):
        assert np.array_equal(o[0, h, 0], v[0, h, 0])
        want = 0.3 * math.fsum(q[0, h, 0, d] * k[0, h, 0, d] for d in range(5))
        assert abs(lse[0, h, 0] - want) <= 1e-15 * max(1.0, abs(want))


def check_causal_prefix(attn):
    """Causal row i equals non-causal attention over keys 0..i."""
    rng = _rng(15)
    S = 8
    q, k, v = (_randn(rng, (1, 1, S, 3)) for _ in range(3))
    o, lse = attn(q, k, v, True, 1.1)
    for i in range(S):
        o2, lse2 = attn(q[:, :, : i + 1], k[:, :, : i + 1], v[:, :, : i + 1], False, 1.1)
        np.testing.assert_allclose(o[0, 0, i], o2[0, 0, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], lse2[0, 0, i], rtol=1e-14, atol=1e-14)


def check_zero_keys_uniform(attn):
    """K = 0 makes every score 0: uniform weights, lse = ln(number of keys)."""
    rng = _rng(16)
    S = 10
    q, v = _randn(rng, (1, 2, S, 4)), _randn(rng, (1, 2, S, 4))
    k = np.zeros((1, 2, S, 4))
    o, lse = attn(q, k, v, False, 0.8)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(S), rtol=1e-15, atol=0)
    o, lse = attn(q, k, v, True, 0.8)
    for i in range(S):
        np.testing.assert_allclose(o[0, :, i], v[0, :, : i + 1].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(i + 1), rtol=0, atol=1e-15)


def check_single_key(attn):
    """S = 1: o = v and lse = scale q.k, with or without the mask."""
    rng = _rng(17)
    q, k, v = (_randn(rng, (2, 3, 1, 6)) for _ in range(3))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.25)
        assert np.array_equal(o, v)
        for b in range(2):
            for h in range(3):
                want = 0.25 * math.fsum(q[b, h, 0, d] * k[b, h, 0, d] for d in range(6))
                assert abs(lse[b, h, 0] - want) <= 1e-15 * max(1.0, abs(want))


def check_closed_form_two_keys(attn):
    """q = (1, 0), k_0 = (1, 0), k_1 = (0, 1), v = (1, 3), scale c:
    row 0 (non-causal) has scores (c, 0): o = (e^c + 3)/(e^c + 1),
    lse = ln(e^c + 1); row 1 (q = (0, 1)) has scores (0, c):
    o = (1 + 3e^c)/(1 + e^c). Causal row 1 keeps both keys; causal row 0 is v_0."""
    c = 0.75
    q = np.array([[1.0, 0.0], [0.0, 1.0]])[None, None]
    k = np.array([[1.0, 0.0], [0.0, 1.0]])[None, None]
    v = np.array([[1.0, -2.0], [3.0, 5.0]])[None, None]
    e = math.exp(c)
    o, lse = attn(q, k, v, False, c)
    np.testing.assert_allclose(o[0, 0, 0], [(e * 1 + 3) / (e + 1), (e * -2 + 5) / (e + 1)], rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [(1 + 3 * e) / (1 + e), (-2 + 5 * e) / (1 + e)], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(e + 1), math.log(1 + e)], rtol=1e-14)
    o, lse = attn(q, k, v, True, c)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, -2.0], rtol=0, atol=0)
    np.testing.assert_allclose(lse[0, 0, 0], c, rtol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], [(1 + 3 * e) / (1 + e), (-2 + 5 * e) / (1 + e)], rtol=1e-14)


def check_powers_of_two(attn):
    """scale = ln 2 and integer scores n_j make every weight a power of two:
    o_i = sum 2^n_j v_j / sum 2^n_j exactly, lse = ln(sum 2^n_j)."""
    q = np.array([[1.0, 2.0, 0.0], [0.0, 1.0, 1.0], [2.0, 0.0, 1.0]])[None, None]
    k = np.array([[1.0, 0.0, 1.0], [0.0, 2.0, 0.0], [1.0, 1.0, 1.0]])[None, None]
    v = np.array([[4.0, 0.0, -1.0], [0.0, 8.0, 3.0], [2.0, 2.0, 5.0]])[None, None]
    n = q[0, 0] @ k[0, 0].T  # integers
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, math.log(2.0))
        for i in range(3):
            cols = range(i + 1) if causal else range(3)
            w = [2.0 ** n[i, j] for j in cols]
            tot = math.fsum(w)
            want = [math.fsum(w[t] * v[0, 0, j, d] for t, j in enumerate(cols)) / tot for d in range(3)]
            np.testing.assert_allclose(o[0, 0, i], want, rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], math.log(tot), rtol=1e-14)


def check_key_shift(attn):
    """Adding u to every key adds scale q_i.u to every score of row i:
    o is unchanged and lse shifts by scale q_i.u (causal or not)."""
    rng = _rng(18)
    q, k, v = (_randn(rng, (1, 2, 7, 4)) for _ in range(3))
    u = _randn(rng, (4,))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.6)
        o2, lse2 = attn(q, k + u, v, causal, 0.6)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse2 - lse, 0.6 * (q @ u), rtol=0, atol=1e-13)


def check_kv_permutation(attn):
    """Non-causal attention is invariant under one permutation of K and V rows."""
    rng = _rng(19)
    q, k, v = (_randn(rng, (2, 2, 11, 5)) for _ in range(3))
    perm = rng.permutation(11)
    o, lse = attn(q, k, v, False, 0.4)
    o2, lse2 = attn(q, k[:, :, perm], v[:, :, perm], False, 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14, atol=1e-14)
    # and it is *not* invariant under permuting K alone (the pairing matters)
    o3, _ = attn(q, k[:, :, perm], v, False, 0.4)
    assert np.abs(o3 - o).max() > 1e-3


def check_brute_force(attn):
    """Plain Python, math.fsum: s = scale * sum_d q k; lse = ln sum exp(s);
    o = sum exp(s) v / sum exp(s). Tiny sizes only."""
    rng = _rng(20)
    B, H, S, D = 1, 2, 6, 3
    q, k, v = (_randn(rng, (B, H, S, D)) for _ in range(3))
    scale = 0.45
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, scale)
        for h in range(H):
            for i in range(S):
                cols = range(i + 1) if causal else range(S)
                s = [scale * math.fsum(q[0, h, i, d] * k[0, h, j, d] for d in range(D)) for j in cols]
                w = [math.exp(x) for x in s]
                tot = math.fsum(w)
                assert abs(lse[0, h, i] - math.log(tot)) <= 1e-13 * max(1.0, abs(math.log(tot)))
                for d in range(D):
                    want = math.fsum(w[t] * v[0, h, j, d] for t, j in enumerate(cols)) / tot
                    assert abs(o[0, h, i, d] - want) <= 1e-13


def check_peaky_rows(attn):
    """One key with score far above the rest: o -> v[j*] with error at most
    2 (S-1) e^{-delta} max|v|. Scores near 1000 also test that the row max is
    subtracted before exponentiating (exp(1000) overflows fp64)."""
    rng = _rng(21)
    S, D = 12, 4
    for delta, base in ((20.0, 0.0), (30.0, 1000.0)):
        q = np.zeros((1, 1, S, D))
        q[0, 0, :, 0] = 1.0
        k = np.zeros((1, 1, S, D))
        k[0, 0, :, 0] = base + rng.uniform(-1, 0, S)  # all scores in [base-1, base]
        jstar = 5
        k[0, 0, jstar, 0] = base + delta
        v = _randn(rng, (1, 1, S, D))
        o, lse = attn(q, k, v, False, 1.0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        bound = 2 * (S - 1) * math.exp(-delta) * np.abs(v).max()
        assert np.abs(o[0, 0] - v[0, 0, jstar]).max() <= bound
        # lse is within ln(1 + (S-1) e^{-delta}) above the top score
        top = base + delta
        assert top <= lse[0, 0, 0] <= top + math.log1p((S - 1) * math.exp(-delta)) + 1e-12


def check_sdpa_float64(attn):
    """Library cross-check: torch's scaled_dot_product_attention in float64 on
    the CPU (a check of the oracle only). lse from torch.logsumexp."""
    import torch
    import torch.nn.functional as F

    rng = _rng(22)
    q, k, v = (_randn(rng, (2, 3, 17, 8)) for _ in range(3))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.35)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.35)
        np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
        s = 0.35 * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(17, 17, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def check_heads_independent(attn):
    """Every (b, h) slice is an independent problem: computing a slice alone
    gives the same rows as computing it inside the full tensor."""
    rng = _rng(23)
    q, k, v = (_randn(rng, (2, 3, 5, 4)) for _ in range(3))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.5)
        for b in range(2):
            for h in range(3):
                sl = (slice(b, b + 1), slice(h, h + 1))
                o1, lse1 = attn(q[sl], k[sl], v[sl], causal, 0.5)
                assert np.array_equal(o1[0, 0], o[b, h])
                assert np.array_equal(lse1[0, 0], lse[b, h])


ALL_CHECKS = [
    check_online_equals_two_pass,
    check_v_ones_gives_ones,
    check_rows_sum_to_one,
    check_causal_row0,
    check_causal_prefix,
    check_zero_keys_uniform,
    check_single_key,
    check_closed_form_two_keys,
    check_powers_of_two,
    check_key_shift,
    check_kv_permutation,
    check_brute_force,
    check_peaky_rows,
    check_sdpa_float64,
    check_heads_independent,
]
