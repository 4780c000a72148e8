"""Checks that pin the oracle's KV-cache form (Sq queries against Sk keys,
queries at the last Sq positions) to facts other than its own formula.

Each check takes `attn_kv(q, k, v, causal, scale) -> (o, lse)` over fp64
numpy arrays, q of shape (B, H, Sq, D) and k, v of shape (B, H, Sk, D), and
raises AssertionError when the fact fails. They run against the real oracle
(tests/test_oracle_kv.py) and against mutated copies of it, where every
planted mistake must trip at least one of them.

None re-types the oracle: the comparisons are a streaming (online-softmax)
evaluation written here, the square causal case evaluated the same way,
closed forms, invariants and a brute-force sum with math.fsum.
"""
from __future__ import annotations

import math

import numpy as np


def _randn(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def online_kv(q, k, v, causal, scale, tile):
    """Online softmax over key tiles (running max, rescaled sum and
    accumulator, one division at the end), queries at positions
    Sk - Sq .. Sk - 1 for the causal mask."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    pos = np.arange(Sq) + (Sk - Sq)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            s_full = scale * (q[b, h] @ k[b, h].T)
            m = np.full(Sq, -np.inf)
            l = np.zeros(Sq)
            acc = np.zeros((Sq, D))
            for start in range(0, Sk, tile):
                cols = np.arange(start, min(start + tile, Sk))
                s = s_full[:, cols].copy()
                if causal:
                    s[pos[:, None] < cols[None, :]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                p = np.exp(s - ref[:, None])
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ v[b, h][cols]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse


def check_kv_online_equals_two_pass(attn_kv):
    rng = np.random.default_rng(31)
    for causal in (False, True):
        for Sq, Sk in ((1, 1), (1, 9), (3, 9), (9, 9), (4, 13)):
            q = _randn(rng, (1, 2, Sq, 4))
            k, v = _randn(rng, (1, 2, Sk, 4)), _randn(rng, (1, 2, Sk, 4))
            o, lse = attn_kv(q, k, v, causal, 0.6)
            for tile in sorted({1, 4, Sk}):
                o2, lse2 = online_kv(q, k, v, causal, 0.6, tile)
                np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def check_kv_noncausal_more_queries_than_keys(attn_kv):
    rng = np.random.default_rng(32)
    q = _randn(rng, (1, 1, 7, 4))
    k, v = _randn(rng, (1, 1, 3, 4)), _randn(rng, (1, 1, 3, 4))
    o, lse = attn_kv(q, k, v, False, 0.8)
    o2, lse2 = online_kv(q, k, v, False, 0.8, 2)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def check_kv_decode_is_square_suffix(attn_kv):
    """The last Sq rows of square causal attention over Sk positions equal the
    KV-cache form given only those Sq queries (the cache holds all Sk keys)."""
    rng = np.random.default_rng(33)
    Sk = 11
    q_all = _randn(rng, (2, 2, Sk, 5))
    k, v = _randn(rng, (2, 2, Sk, 5)), _randn(rng, (2, 2, Sk, 5))
    o_sq, lse_sq = online_kv(q_all, k, v, True, 0.5, 3)  # Sq = Sk: the square case
    for Sq in (1, 2, 5, Sk):
        o, lse = attn_kv(q_all[:, :, Sk - Sq:].copy(), k, v, True, 0.5)
        np.testing.assert_allclose(o, o_sq[:, :, Sk - Sq:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_sq[:, :, Sk - Sq:], rtol=1e-12, atol=1e-12)


def check_kv_v_ones(attn_kv):
    rng = np.random.default_rng(34)
    q = _randn(rng, (1, 2, 4, 8))
    k = _randn(rng, (1, 2, 10, 8))
    for causal in (False, True):
        o, _ = attn_kv(q, k, np.ones((1, 2, 10, 8)), causal, 0.5)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)


def check_kv_zero_keys_uniform(attn_kv):
    """K = 0: every visible key scores 0, so O is the mean of the visible V
    rows and lse = ln(number of visible keys), for query i of Sq against Sk:
    Sk keys, or i + Sk - Sq + 1 under the causal mask."""
    rng = np.random.default_rng(35)
    Sq, Sk = 4, 9
    q = _randn(rng, (1, 1, Sq, 3))
    k = np.zeros((1, 1, Sk, 3))
    v = _randn(rng, (1, 1, Sk, 3))
    o, lse = attn_kv(q, k, v, False, 0.9)
    for i in range(Sq):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(Sk)) < 1e-14
    o, lse = attn_kv(q, k, v, True, 0.9)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-14


def check_kv_single_key(attn_kv):
    rng = np.random.default_rng(36)
    q = _randn(rng, (2, 2, 1, 6))
    k, v = _randn(rng, (2, 2, 1, 6)), _randn(rng, (2, 2, 1, 6))
    for causal in (False, True):
        o, lse = attn_kv(q, k, v, causal, 0.4)
        np.testing.assert_array_equal(o, v)
        for b in range(2):
            for h in range(2):
                dot = math.fsum(q[b, h, 0, d] * k[b, h, 0, d] for d in range(6))
                assert abs(lse[b, h, 0] - 0.4 * dot) < 1e-13


def check_kv_permutation(attn_kv):
    rng = np.random.default_rng(37)
    q = _randn(rng, (1, 2, 3, 5))
    k, v = _randn(rng, (1, 2, 12, 5)), _randn(rng, (1, 2, 12, 5))
    perm = rng.permutation(12)
    o1, lse1 = attn_kv(q, k, v, False, 0.7)
    o2, lse2 = attn_kv(q, k[:, :, perm].copy(), v[:, :, perm].copy(), False, 0.7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-13, atol=1e-13)


def check_kv_brute_force(attn_kv):
    """Every output element as math.fsum sums of math.exp terms over the
    visible keys, on a tiny case with several batches and heads."""
    rng = np.random.default_rng(38)
    B, H, Sq, Sk, D = 2, 2, 3, 5, 3
    q = _randn(rng, (B, H, Sq, D))
    k, v = _randn(rng, (B, H, Sk, D)), _randn(rng, (B, H, Sk, D))
    for causal in (False, True):
        o, lse = attn_kv(q, k, v, causal, 1.1)
        for b in range(B):
            for h in range(H):
                for i in range(Sq):
                    keys = range(i + Sk - Sq + 1) if causal else range(Sk)
                    s = [1.1 * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in keys]
                    mx = max(s)
                    e = [math.exp(x - mx) for x in s]
                    l = math.fsum(e)
                    assert abs(lse[b, h, i] - (mx + math.log(l))) < 1e-12
                    for d in range(D):
                        ref = math.fsum(e[t] * v[b, h, j, d] for t, j in enumerate(keys)) / l
                        assert abs(o[b, h, i, d] - ref) < 1e-12


ALL_KV_CHECKS = [
    check_kv_online_equals_two_pass,
    check_kv_noncausal_more_queries_than_keys,
    check_kv_decode_is_square_suffix,
    check_kv_v_ones,
    check_kv_zero_keys_uniform,
    check_kv_single_key,
    check_kv_permutation,
    check_kv_brute_force,
]
