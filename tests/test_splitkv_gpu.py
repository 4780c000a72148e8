"""Split-KV (decoding / KV-cache) path vs the fp64 oracle's KV-cache form.

Sq queries against Sk keys per head, the queries being the last Sq
positions (causal keeps key j for query i iff j <= i + Sk - Sq). Every
output is compared at the parity bar of test_parity_gpu (max |dO| <= 2e-3
fp16 / 1.6e-2 bf16, lse relative error <= 1e-4), over head dims, dtypes,
ragged lengths, split counts (including more chunks than key tiles, and 0 =
the library's choice) and query counts that span several 32-row blocks.
"""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import oracle
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, scale, n_split, workspace=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.attention_splitkv(qd, kd, vd, causal=causal, scale=scale, n_split=n_split,
                                  workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _oracle(q, k, v, causal, scale):
    return oracle.attention_kv_f64(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                   causal, scale)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_splitkv_shapes(D, dtype):
    cases = [(1, 1), (1, 31), (1, 33), (1, 1000), (3, 257), (32, 32), (33, 100), (70, 300),
             (5, 2)]  # the last has Sq > Sk (non-causal only)
    for Sq, Sk in cases:
        for causal in (False, True):
            if causal and Sq > Sk:
                continue
            for n_split in (1, 3, 0, 64):
                w = wl.DecodeWorkload("t", 2, 2, Sq, Sk, D, dtype, causal)
                what = f"splitkv D={D} {dtype} Sq={Sq} Sk={Sk} causal={causal} n_split={n_split}"
                announce(what)
                q, k, v = wl.make_qkv_decode(w, seed=Sq * 1000 + Sk)
                o, lse = _run(q, k, v, causal, w.scale, n_split)
                o_ref, lse_ref = _oracle(q, k, v, causal, w.scale)
                assert_parity(o, lse, o_ref, lse_ref, dtype, what)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_splitkv_negative_scale(D, dtype):
    """scale = -1/sqrt(D) (and -3/sqrt(D) with Q and K x3): every output
    against the oracle, causal and not, several split counts."""
    for mult in (1.0, 3.0):
        for causal in (False, True):
            for n_split in (1, 3, 0):
                w = wl.DecodeWorkload("neg", 2, 2, 17, 700, D, dtype, causal, qk_mult=mult)
                scale = -mult / D ** 0.5
                what = (f"splitkv negative scale {scale:.4f} D={D} {dtype} causal={causal} "
                        f"n_split={n_split}")
                announce(what)
                q, k, v = wl.make_qkv_decode(w, seed=D + n_split)
                o, lse = _run(q, k, v, causal, scale, n_split)
                o_ref, lse_ref = _oracle(q, k, v, causal, scale)
                assert_parity(o, lse, o_ref, lse_ref, dtype, what)


@pytest.mark.parametrize("w", wl.DECODE, ids=lambda w: w.name)
def test_splitkv_benchmark_shapes(w):
    """The benchmark decoding shapes at full size, every output (the oracle
    is cheap here: few queries)."""
    announce(f"splitkv {w}")
    q, k, v = wl.make_qkv_decode(w, seed=0)
    o, lse = _run(q, k, v, w.causal, w.scale, 0)
    o_ref, lse_ref = _oracle(q, k, v, w.causal, w.scale)
    assert_parity(o, lse, o_ref, lse_ref, w.dtype, w.name)


def test_splitkv_equals_square_path_when_lengths_match():
    """Sq = Sk is the square problem: both entry points agree within the bar."""
    w = wl.Workload("sq", 1, 4, 300, 128, "f16", True)
    q, k, v = wl.make_qkv(w, seed=9)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o1, l1 = fa.attention(qd, kd, vd, causal=True, scale=w.scale)
    o2, l2 = fa.attention_splitkv(qd, kd, vd, causal=True, scale=w.scale, n_split=4)
    torch.cuda.synchronize()
    assert (o1.double() - o2.double()).abs().max().item() <= 2e-3
    assert ((l1 - l2).abs() / l1.abs().clamp_min(1)).max().item() <= 1e-4


def test_splitkv_peaky_and_rising_scores():
    """Large logits (Q and K x3) and scores that climb along the keys, so the
    chunks' maxima differ by far more than fp32 exp can span."""
    for qk_mult in (3.0,):
        w = wl.DecodeWorkload("peaky", 1, 4, 4, 5000, 128, "bf16", False, qk_mult=qk_mult)
        q, k, v = wl.make_qkv_decode(w, seed=4)
        o, lse = _run(q, k, v, False, w.scale, 7)
        o_ref, lse_ref = _oracle(q, k, v, False, w.scale)
        assert_parity(o, lse, o_ref, lse_ref, "bf16", "splitkv peaky")
    g = torch.Generator().manual_seed(5)
    Sq, Sk, D = 3, 2000, 128
    q = torch.randn(1, 2, Sq, D, generator=g) * 0.25
    k = torch.randn(1, 2, Sk, D, generator=g) * 0.25
    v = torch.randn(1, 2, Sk, D, generator=g)
    q[..., 0] = 8.0
    k[..., 0] = torch.arange(Sk, dtype=torch.float32) / Sk * (80.0 / (8.0 * 1.4427 / D ** 0.5))
    q, k, v = q.half(), k.half(), v.half()
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, 1.0 / D ** 0.5, 9)
        o_ref, lse_ref = _oracle(q, k, v, causal, 1.0 / D ** 0.5)
        assert_parity(o, lse, o_ref, lse_ref, "f16", f"splitkv rising causal={causal}")


def test_splitkv_deterministic_and_workspace_reuse():
    w = wl.DecodeWorkload("det", 2, 3, 2, 777, 64, "f16", True)
    q, k, v = wl.make_qkv_decode(w, seed=1)
    need = fa.fa2_splitkv_workspace_bytes(2, 3, 2, 777, 64, 5)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    a = _run(q, k, v, True, w.scale, 5, workspace=ws)
    b = _run(q, k, v, True, w.scale, 5, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # nothing past the documented size is written
    assert (ws[need:] == 0x5A).all()


def test_splitkv_outputs_leave_neighbours_untouched():
    B, H, Sq, Sk, D = 2, 2, 3, 300, 128
    w = wl.DecodeWorkload("guard", B, H, Sq, Sk, D, "bf16", True)
    q, k, v = (x.to(DEV) for x in wl.make_qkv_decode(w, seed=2))
    g = 4096
    n, nl = B * H * Sq * D, B * H * Sq
    obuf = torch.full((g + n + g,), 7.0, dtype=q.dtype, device=DEV)
    lbuf = torch.full((g + nl + g,), -3.0, dtype=torch.float32, device=DEV)
    o = obuf[g:g + n].view(q.shape)
    lse = lbuf[g:g + nl].view(B, H, Sq)
    fa.attention_splitkv(q, k, v, causal=True, scale=w.scale, n_split=3, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:g] == 7.0).all() and (obuf[g + n:] == 7.0).all()
    assert (lbuf[:g] == -3.0).all() and (lbuf[g + nl:] == -3.0).all()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_splitkv_rejects_short_workspace():
    w = wl.DecodeWorkload("ws", 1, 1, 1, 64, 64, "f16", False)
    q, k, v = (x.to(DEV) for x in wl.make_qkv_decode(w, seed=3))
    ws = torch.empty((16,), dtype=torch.uint8, device=DEV)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention_splitkv(q, k, v, n_split=2, workspace=ws)
    assert e.value.status == fa.FA2_ERR_WORKSPACE
