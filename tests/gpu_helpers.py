"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle
on the same rounded inputs, and compare at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import flashattention_tiled_amd as fa
import oracle
from workloads import TOLERANCE_LSE_REL, TOLERANCE_O

DEV = "cuda:0"


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, causal, scale):
    """q, k, v: CPU tensors (fp16/bf16). Returns (o, lse) on the CPU."""
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def widen(x) -> np.ndarray:
    return x.double().numpy()


def oracle_full(q, k, v, causal, scale):
    return oracle.attention_f64(widen(q), widen(k), widen(v), causal, scale)


def oracle_rows(q, k, v, rows, causal, scale):
    return oracle.attention_rows_f64(widen(q), widen(k), widen(v), rows, causal, scale)


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    """(max |O_gpu - O_ref|, max |lse_gpu - lse_ref| / max(|lse_ref|, 1))."""
    o_err = np.abs(o_gpu.double().numpy().reshape(o_ref.shape) - o_ref).max()
    lg = lse_gpu.double().numpy().reshape(lse_ref.shape)
    lse_err = (np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max()
    return float(o_err), float(lse_err)


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str):
    assert torch.isfinite(o_gpu.float()).all(), f"{what}: non-finite O"
    assert torch.isfinite(lse_gpu).all(), f"{what}: non-finite lse"
    o_err, lse_err = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    print(f"[parity] {what}: max|dO|={o_err:.3e} (tol {TOLERANCE_O[dtype]:.1e}) "
          f"lse_rel={lse_err:.3e} (tol {TOLERANCE_LSE_REL:.0e})", flush=True)
    assert o_err <= TOLERANCE_O[dtype], f"{what}: max|dO| {o_err:.3e} > {TOLERANCE_O[dtype]}"
    assert lse_err <= TOLERANCE_LSE_REL, f"{what}: lse rel err {lse_err:.3e} > {TOLERANCE_LSE_REL}"


def sample_rows(B, H, S, n_random=48, seed=0, tile=128):
    """Flat row indices (b*H + h)*S + i: edges, tile boundaries, the ragged
    tail and random rows, spread over several heads."""
    rng = np.random.default_rng(seed)
    heads = sorted({0, B * H - 1, *rng.integers(0, B * H, size=3).tolist()})
    fixed = {0, 1, 2, S - 1, S - 2, S // 2}
    for t in (tile - 1, tile, tile + 1, 2 * tile - 1, 2 * tile):
        if t < S:
            fixed.add(t)
    rows = set()
    for bh in heads:
        for i in fixed:
            if 0 <= i < S:
                rows.add(bh * S + i)
    rows.update((rng.integers(0, B * H) * S + rng.integers(0, S, size=n_random)).tolist())
    return np.array(sorted(rows), dtype=np.int64)
