"""Pins of the FP8 path's tolerance (oracle.attention_fp8_bound_f64), on the CPU.

The bound is a forward error analysis of attention computed with FP8
products (sums within eps of exact, relative to the sum of |terms|) and P
rounded to e4m3 as 2^(t - m + p_exp) under a lazily raised reference max m.
It is pinned here against an emulation of exactly that arithmetic in
fp64, written from the description of the algorithm, not from the bound's
formula: logits perturbed anywhere within the products' error (at random,
and pushed all one way), m moved tile by tile as the kernel moves it, P
rounded to e4m3 by torch's float8_e4m3fn cast, the sums of P V and of P
perturbed within eps, O rounded once to fp16 or bf16. Every emulated output
must stay within the bound, over shapes from one key to a few hundred,
peaky, flat and one-hot rows, negative scales and causal masking. The
emulation reaches a sizable fraction of the bound in its worst cases, so a
bound a few times too tight fails here (checked with a shrunk bound).
Also: the bound's O and lse are exactly the oracle's attention_f64.
"""
import math

import numpy as np
import pytest
import torch

import oracle

EPS = 2.0 ** -11
P_EXP = 6.0
HEADROOM = 2.75
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TILE = 8  # keys per tile in the emulation (the kernel's are 64; the rule is the same)
LOG2E = 1.4426950408889634


def _e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _round_out(x: np.ndarray, dt: str) -> np.ndarray:
    td = torch.float16 if dt == "f16" else torch.bfloat16
    return torch.from_numpy(x).to(td).to(torch.float64).numpy()


def emulate(q, k, v, causal, scale, dt, rng, mode):
    """The FP8 path's arithmetic, row by row, with the products' errors
    chosen by `mode`: "random" (uniform within the bound), "push" (every
    logit error and sum error pushed to the side that raises O[..., 0]),
    or "zero"."""
    B, H, S, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, S))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                n = i + 1 if causal else S
                qi, kk, vv = q[b, h, i], k[b, h, :n], v[b, h, :n]
                s = scale * (kk @ qi)
                a = abs(scale) * (np.abs(kk * qi).sum(-1))
                if mode == "random":
                    u = rng.uniform(-1, 1, n)
                elif mode == "push":
                    o0 = (np.exp(s - s.max()) @ vv[:, 0]) / np.exp(s - s.max()).sum()
                    u = np.sign(vv[:, 0] - o0)
                else:
                    u = np.zeros(n)
                t = (s + EPS * a * u) * LOG2E  # the logits the kernel sees
                # the reference max: tile 0's row max, raised to a tile's max
                # when that passes m + HEADROOM; P of each tile against the m
                # of its time, later rescaled to the final m
                m = t[:TILE].max()
                p8 = np.empty(n)
                p_fp = np.empty(n)
                m_at = np.empty(n)
                for t0 in range(0, n, TILE):
                    sl = slice(t0, min(n, t0 + TILE))
                    if t[sl].max() > m + HEADROOM:
                        m = t[sl].max()
                    p = np.exp2(t[sl] - m + P_EXP)
                    p_fp[sl] = p
                    p8[sl] = _e4m3(p)
                    m_at[sl] = m
                scale_back = np.exp2(m_at - m)  # the rescale by 2^(m_old - m_new)
                w8 = p8 * scale_back
                num = w8 @ vv
                den = w8.sum()
                e_num = EPS * (np.abs(w8) @ np.abs(vv))
                e_den = EPS * den
                if mode == "push":
                    num = num + e_num * np.where(np.arange(D) == 0, 1.0, 0.0)
                    den = den - e_den
                elif mode == "random":
                    num = num + e_num * rng.uniform(-1, 1, D)
                    den = den + e_den * rng.uniform(-1, 1)
                o[b, h, i] = _round_out(num / den, dt)
                lse[b, h, i] = (m + math.log2((p_fp * scale_back).sum()) - P_EXP) / LOG2E
    return o, lse


def _inputs(B, H, S, D, rng, mult=1.0, descale=1 / 32):
    """e4m3 inputs: N(0, mult^2) values / descale, cast once, times descale."""
    def one():
        x = rng.standard_normal((B, H, S, D)) * mult / descale
        return _e4m3(np.clip(x, -448, 448)) * descale
    return one(), one(), one()


CASES = [
    # (B, H, S, D, causal, scale sign, q/k multiplier, dtype)
    (1, 2, 1, 16, False, 1, 1.0, "f16"),
    (1, 2, 37, 16, True, 1, 1.0, "f16"),
    (1, 1, 200, 32, False, 1, 1.0, "bf16"),
    (1, 1, 150, 16, True, 1, 3.0, "bf16"),
    (1, 1, 120, 16, False, 1, 8.0, "f16"),   # near one-hot rows
    (1, 1, 120, 16, False, -1, 3.0, "f16"),  # negative scale
    (2, 1, 64, 16, True, -1, 1.0, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_emulated_fp8_within_bound(case):
    B, H, S, D, causal, sign, mult, dt = case
    rng = np.random.default_rng(S * 7 + D)
    q, k, v = _inputs(B, H, S, D, rng, mult)
    scale = sign / math.sqrt(D)
    o_ref, lse_ref, bo, bl = oracle.attention_fp8_bound_f64(q, k, v, causal, scale, EPS, P_EXP,
                                                            U_OUT[dt])
    o_plain, lse_plain = oracle.attention_f64(q, k, v, causal, scale)
    assert np.array_equal(o_ref, o_plain) and np.array_equal(lse_ref, lse_plain)
    assert (bo > 0).all() and (bl > 0).all()
    for mode in ("zero", "random", "push"):
        o, lse = emulate(q, k, v, causal, scale, dt, rng, mode)
        ratio_o = (np.abs(o - o_ref) / bo).max()
        ratio_l = (np.abs(lse - lse_ref) / bl).max()
        print(f"{case} {mode}: max |dO| / bound {ratio_o:.3f}, max |dlse| / bound {ratio_l:.3f}")
        assert ratio_o <= 1.0 and ratio_l <= 1.0, (mode, ratio_o, ratio_l)


def test_flat_rows():
    """K = 0: every score equal, so every P is 2^p_exp exactly and the only
    error left is the output rounding; the bound allows it."""
    rng = np.random.default_rng(5)
    q, _, v = _inputs(1, 1, 100, 16, rng)
    k = np.zeros_like(q)
    o_ref, lse_ref, bo, bl = oracle.attention_fp8_bound_f64(q, k, v, False, 0.25, EPS, P_EXP,
                                                            U_OUT["f16"])
    o, lse = emulate(q, k, v, False, 0.25, "f16", rng, "zero")
    assert np.allclose(lse_ref, math.log(100)) and (np.abs(lse - lse_ref) <= bl).all()
    assert (np.abs(o - o_ref) <= bo).all()


def test_bound_is_not_vacuous():
    """The worst emulated cases come within a factor of a few of the bound:
    a bound a quarter as large fails somewhere (O or lse)."""
    worst = 0.0
    for case in CASES:
        B, H, S, D, causal, sign, mult, dt = case
        rng = np.random.default_rng(S * 7 + D)
        q, k, v = _inputs(B, H, S, D, rng, mult)
        scale = sign / math.sqrt(D)
        o_ref, lse_ref, bo, bl = oracle.attention_fp8_bound_f64(q, k, v, causal, scale, EPS,
                                                                P_EXP, U_OUT[dt])
        o, lse = emulate(q, k, v, causal, scale, dt, rng, "push")
        worst = max(worst, (np.abs(o - o_ref) / bo).max(), (np.abs(lse - lse_ref) / bl).max())
    print(f"largest emulated error / bound: {worst:.3f}")
    assert worst > 0.25
