"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Tolerances (written here, applied to every case): max |O_gpu - O_ref| <= 2e-3
for fp16 output and <= 1.6e-2 for bf16 output; lse relative error
|lse_gpu - lse_ref| / max(|lse_ref|, 1) <= 1e-4.

Small sizes compare every output; the full benchmark shapes compare sampled
rows (edges, tile boundaries, the ragged tail, random rows) that the oracle
computes one by one, in the same launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import (DEV, announce, assert_parity, oracle_full, oracle_rows, run_gpu,
                         sample_rows)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# the tiny exact configuration, every output, three seeds
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("w", wl.TINY, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_full(w, seed):
    announce(f"tiny {w} seed={seed}")
    q, k, v = wl.make_qkv(w, seed)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle_full(q, k, v, w.causal, w.scale)
    assert_parity(o, lse, o_ref, lse_ref, w.dtype, f"{w.name} seed {seed}")


# ---------------------------------------------------------------------------
# small shapes spanning several tiles and ragged tails, every output
# ---------------------------------------------------------------------------
SMALL_S = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 257, 383]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes_full(D, dtype, causal):
    for S in SMALL_S:
        w = wl.Workload(f"small_S{S}", 1, 2, S, D, dtype, causal)
        announce(f"small {w}")
        q, k, v = wl.make_qkv(w, seed=S)
        o, lse = run_gpu(q, k, v, causal, w.scale)
        o_ref, lse_ref = oracle_full(q, k, v, causal, w.scale)
        assert_parity(o, lse, o_ref, lse_ref, dtype, w.name + f" D{D} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_batch_heads_full(dtype):
    """Several batches and heads with a ragged S: every (b, h) slice is checked."""
    for causal in (False, True):
        w = wl.Workload("multi_bh", 3, 5, 301, 128, dtype, causal)
        announce(f"multi {w}")
        q, k, v = wl.make_qkv(w, seed=7)
        o, lse = run_gpu(q, k, v, causal, w.scale)
        o_ref, lse_ref = oracle_full(q, k, v, causal, w.scale)
        assert_parity(o, lse, o_ref, lse_ref, dtype, f"multi_bh causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_peaky_small_full(dtype):
    """Q and K scaled x3 (peaky softmax rows), as in the long-prefill workload."""
    w = wl.Workload("peaky", 1, 4, 700, 128, dtype, False, qk_mult=3.0)
    announce(f"peaky {w}")
    q, k, v = wl.make_qkv(w, seed=3)
    o, lse = run_gpu(q, k, v, False, w.scale)
    o_ref, lse_ref = oracle_full(q, k, v, False, w.scale)
    assert_parity(o, lse, o_ref, lse_ref, dtype, "peaky small")


def _ramp_inputs(S, D, dtype, direction, seed):
    """Scores that climb steeply along the keys (direction +1) or fall
    (direction -1): every query has q[0] = 8 and key j has k[j, 0] growing
    linearly with j, so the base-2 logit of the last keys exceeds that of the
    first tile by about 60. Other components are small N(0, 0.25^2) noise;
    v is N(0, 1). Rounded once to the dtype, like every other input."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(1, 2, S, D, generator=g) * 0.25
    k = torch.randn(1, 2, S, D, generator=g) * 0.25
    v = torch.randn(1, 2, S, D, generator=g)
    c = 1.4426950408889634 / D ** 0.5
    amp = 60.0 / (8.0 * c)
    ramp = torch.arange(S, dtype=torch.float32) / S * amp
    q[..., 0] = 8.0
    k[..., 0] = ramp if direction > 0 else ramp.flip(0)
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    return q.to(td), k.to(td), v.to(td)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rising_scores_force_rescale(D, dtype):
    """Later key tiles score far above the first one, so the kernel's lazy
    reference max must be raised mid-sequence (the redo path of a tile whose
    row sum of P passes 2^12), repeatedly; a falling ramp never raises it."""
    for causal in (False, True):
        for direction in (1, -1):
            S = 700
            announce(f"ramp D={D} {dtype} causal={causal} direction={direction}")
            q, k, v = _ramp_inputs(S, D, dtype, direction, seed=11 + D)
            scale = 1.0 / D ** 0.5
            o, lse = run_gpu(q, k, v, causal, scale)
            o_ref, lse_ref = oracle_full(q, k, v, causal, scale)
            assert_parity(o, lse, o_ref, lse_ref, dtype,
                          f"ramp D{D} {dtype} causal={causal} dir={direction}")


def test_scale_values():
    """Scale 0 (uniform weights), a large scale, and a non-default value."""
    for scale in (0.0, 0.5, 1.0 / 3.0):
        w = wl.Workload("scales", 1, 2, 190, 64, "f16", True)
        announce(f"scale={scale} {w}")
        q, k, v = wl.make_qkv(w, seed=5)
        o, lse = run_gpu(q, k, v, True, scale)
        o_ref, lse_ref = oracle_full(q, k, v, True, scale)
        assert_parity(o, lse, o_ref, lse_ref, "f16", f"scale {scale}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_negative_scale(D, dtype):
    """A negative scale (here -1/sqrt(D), and -3/sqrt(D) on peaky inputs)
    reverses the order of the scores: the row max is then the scale times
    the smallest dot product, which the kernel's first-tile max and its
    rescale redo must both take in the scaled domain. Every output, causal
    and not, ragged S over several tiles."""
    for causal in (False, True):
        for mult, S in ((1.0, 383), (3.0, 700)):
            w = wl.Workload("neg", 1, 2, S, D, dtype, causal, qk_mult=mult)
            scale = -mult / D ** 0.5
            announce(f"negative scale {scale:.4f} {w}")
            q, k, v = wl.make_qkv(w, seed=D + S)
            o, lse = run_gpu(q, k, v, causal, scale)
            o_ref, lse_ref = oracle_full(q, k, v, causal, scale)
            assert_parity(o, lse, o_ref, lse_ref, dtype,
                          f"scale {scale:.4f} D{D} {dtype} causal={causal} x{mult}")


def test_negative_scale_falling_ramp():
    """The ramp inputs above with a negative scale: the scores now climb
    along the keys where the positive scale made them fall, forcing the
    lazy reference max up tile after tile."""
    for D in (64, 128, 256):
        for causal in (False, True):
            announce(f"negative-scale ramp D={D} causal={causal}")
            q, k, v = _ramp_inputs(700, D, "f16", -1, seed=3 + D)
            scale = -1.0 / D ** 0.5
            o, lse = run_gpu(q, k, v, causal, scale)
            o_ref, lse_ref = oracle_full(q, k, v, causal, scale)
            assert_parity(o, lse, o_ref, lse_ref, "f16", f"neg ramp D{D} causal={causal}")


# ---------------------------------------------------------------------------
# the benchmark shapes at full size, sampled rows
# ---------------------------------------------------------------------------
FULL = wl.SWEEP + wl.LLM_LAYER + [wl.LONG_PREFILL, wl.RAGGED_D256, wl.ONE_GPU_SHARE]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_size_sampled(w):
    announce(f"full-size {w}")
    q, k, v = wl.make_qkv(w, seed=0)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rows = sample_rows(w.B, w.H, w.S)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, w.causal, w.scale)
    o_s = o.reshape(-1, w.D)[torch.from_numpy(rows)]
    lse_s = lse.reshape(-1)[torch.from_numpy(rows)]
    assert_parity(o_s, lse_s, o_ref, lse_ref, w.dtype, f"{w.name} ({len(rows)} rows)")
    if fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, int(w.causal)) > 0:
        # attention() split this shape's keys: check the unsplit launch too
        qd, kd, vd = (x.to(DEV) for x in (q, k, v))
        o1, lse1 = fa.attention(qd, kd, vd, causal=w.causal, scale=w.scale, balanced=False)
        torch.cuda.synchronize()
        o_s = o1.cpu().reshape(-1, w.D)[torch.from_numpy(rows)]
        lse_s = lse1.cpu().reshape(-1)[torch.from_numpy(rows)]
        assert_parity(o_s, lse_s, o_ref, lse_ref, w.dtype, f"{w.name} unsplit ({len(rows)} rows)")


@pytest.mark.parametrize("S", [8192, 8223, 12001])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d64_long_sequence_tile(S, dtype, causal):
    """D = 64 switches to its long-sequence tile (32 keys, four waves per
    SIMD) at S >= 8192: sampled rows, including the ragged tail, against the
    oracle, and the peaky rising-score case that forces the lazy rescale."""
    w = wl.Workload("d64_long", 1, 3, S, 64, dtype, causal)
    announce(f"d64 long tile S={S} {dtype} causal={causal}")
    q, k, v = wl.make_qkv(w, seed=S)
    o, lse = run_gpu(q, k, v, causal, w.scale)
    rows = sample_rows(w.B, w.H, S, seed=S, tile=128)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, causal, w.scale)
    o_s = o.reshape(-1, 64)[torch.from_numpy(rows)]
    lse_s = lse.reshape(-1)[torch.from_numpy(rows)]
    assert_parity(o_s, lse_s, o_ref, lse_ref, dtype, f"d64 long S={S} ({len(rows)} rows)")
    if S == 8223:
        q2, k2, v2 = _ramp_inputs(S, 64, dtype, +1, seed=1)
        o2, lse2 = run_gpu(q2, k2, v2, causal, w.scale)
        rows2 = sample_rows(1, 2, S, seed=S + 1, tile=128)
        o_ref2, lse_ref2 = oracle_rows(q2, k2, v2, rows2, causal, w.scale)
        assert_parity(o2.reshape(-1, 64)[torch.from_numpy(rows2)],
                      lse2.reshape(-1)[torch.from_numpy(rows2)], o_ref2, lse_ref2, dtype,
                      f"d64 long rising scores S={S}")
