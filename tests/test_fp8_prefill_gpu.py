"""fa2_fwd_fp8 (FP8 e4m3 Q, K, V on the FP8 matrix cores) against the fp64
oracle on the dequantized inputs, every output, at the FP8 path's derived
tolerance: oracle.attention_fp8_bound_f64 bounds, per output, what FP8
products (sum accuracy workloads.FP8_MFMA_SUM_REL, measured in
test_fp8_mfma_gpu.py), P rounded to e4m3 as 2^(t - m + 6) under the lazily
moved reference max, and the final rounding to fp16 / bf16 can change; the
derivation is in oracle/attn_oracle.c and its pins in
test_oracle_fp8_bound.py. Both |dO| <= bound_o and |dlse| <= bound_lse must
hold for every element."""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import oracle
import workloads as wl
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu

P_EXP = 6.0
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _check(w, seed=0, scale=None, label=""):
    scale = w.scale if scale is None else scale
    q8, k8, v8 = wl.make_qkv_fp8(w, seed)
    dq, dk, dv = wl.fp8_descales(w)
    out_dt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    o, lse = fa.attention_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=w.causal, scale=scale,
                              q_descale=dq, k_descale=dk, v_descale=dv, out_dtype=out_dt)
    torch.cuda.synchronize()
    qn, kn, vn = (wl.dequantize_fp8(x, d).numpy() for x, d in ((q8, dq), (k8, dk), (v8, dv)))
    o_ref, lse_ref, bo, bl = oracle.attention_fp8_bound_f64(qn, kn, vn, w.causal, scale,
                                                            wl.FP8_MFMA_SUM_REL, P_EXP,
                                                            U_OUT[w.dtype])
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all(), label
    do = np.abs(og - o_ref)
    dl = np.abs(lg - lse_ref)
    r_o, r_l = float((do / bo).max()), float((dl / bl).max())
    print(f"[fp8 parity] {label} {w}: max|dO| {do.max():.3e} (rms {np.sqrt((do ** 2).mean()):.2e}), "
          f"max|dO|/bound {r_o:.3f}; max|dlse| {dl.max():.3e}, /bound {r_l:.3f}", flush=True)
    assert r_o <= 1.0, f"{label}: O outside the FP8 bound ({r_o:.3f})"
    assert r_l <= 1.0, f"{label}: lse outside the FP8 bound ({r_l:.3f})"
    return do.max(), r_o


SMALL_S = [1, 2, 63, 64, 65, 129, 200, 383]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_small_shapes(D, dtype, causal):
    for S in SMALL_S:
        w = wl.Workload("fp8_small", 1, 2, S, D, dtype, causal)
        announce(f"fp8 {w}")
        _check(w, seed=S, label=f"S={S}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_fp8_peaky_and_negative_scale(D):
    for causal in (False, True):
        w = wl.Workload("fp8_peaky", 1, 3, 700, D, "bf16", causal, qk_mult=3.0)
        announce(f"fp8 peaky {w}")
        _check(w, seed=D, label="peaky x3")
        w = wl.Workload("fp8_neg", 2, 2, 301, D, "f16", causal)
        announce(f"fp8 negative scale {w}")
        _check(w, seed=D + 1, scale=-w.scale, label="negative scale")


def test_fp8_rising_scores_force_rescale():
    """Scores climbing steeply along the keys make the kernel raise its
    reference max again and again (the redo on a tile whose row max passes
    m + 2.75): q[0] = 8 for every query, k[j, 0] growing with j."""
    for causal in (False, True):
        S, D = 700, 128
        g = torch.Generator().manual_seed(3)
        q = torch.randn(1, 2, S, D, generator=g) * 0.25
        k = torch.randn(1, 2, S, D, generator=g) * 0.25
        v = torch.randn(1, 2, S, D, generator=g)
        q[..., 0] = 8.0
        k[..., 0] = torch.linspace(0, 60.0 / (8.0 * 1.4427 / D ** 0.5), S)
        d = 1.0 / 32
        q8, k8, v8 = (torch.clamp(x / d, -448, 448).to(torch.float8_e4m3fn) for x in (q, k, v))
        announce(f"fp8 rising scores causal={causal}")
        o, lse = fa.attention_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=causal,
                                  scale=1 / D ** 0.5, q_descale=d, k_descale=d, v_descale=d)
        torch.cuda.synchronize()
        qn, kn, vn = (wl.dequantize_fp8(x, d).numpy() for x in (q8, k8, v8))
        o_ref, lse_ref, bo, bl = oracle.attention_fp8_bound_f64(qn, kn, vn, causal, 1 / D ** 0.5,
                                                                wl.FP8_MFMA_SUM_REL, P_EXP,
                                                                U_OUT["f16"])
        do = np.abs(o.cpu().double().numpy() - o_ref)
        dl = np.abs(lse.cpu().double().numpy() - lse_ref)
        print(f"[fp8 parity] rising causal={causal}: max|dO|/bound {(do / bo).max():.3f}, "
              f"max|dlse|/bound {(dl / bl).max():.3f}", flush=True)
        assert (do <= bo).all() and (dl <= bl).all()


def test_fp8_ragged_d256_every_row():
    """B=4, H=16, S=4097, D=256, bf16 out, causal (the ragged benchmark
    shape, on the unpipelined D = 256 loop): every output within the bound."""
    w = wl.Workload("fp8_ragged_d256", 4, 16, 4097, 256, "bf16", True)
    announce(f"fp8 ragged D=256 {w}")
    _check(w, seed=0, label="ragged D=256")


def test_fp8_headline_shape_every_row():
    """B=2, H=16, S=8192, D=128, causal: every output of the benchmark
    shape within the bound."""
    w = wl.Workload("fp8_headline", 2, 16, 8192, 128, "f16", True)
    announce(f"fp8 headline {w}")
    _check(w, seed=0, label="headline")


def test_fp8_validation():
    announce("fp8 validation")
    x = torch.zeros(1, 1, 64, 96, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention_fp8(x, x, x)
    assert e.value.status == fa.FA2_ERR_HEADDIM
    y = torch.zeros(1, 1, 64, 64, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention_fp8(y, y, y, k_descale=0.0)
    assert e.value.status == fa.FA2_ERR_SCALE
