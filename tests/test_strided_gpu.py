"""Strided tensors through fa2_fwd_strided: the same results as fa2_fwd on
contiguous copies, bit for bit (only the addressing differs), parity with
the oracle, and nothing written outside o's rows.

Layouts: (B, S, H, D) views (a transposed projection output), the three
views of one packed (B, S, 3, H, D) QKV buffer, a K and V of one head shared
by all heads (head stride 0), rows padded to D + 64 elements, and Q's rows
apart by another stride than K's and V's (a (B, S, H, D) view of Q beside
K and V with padded rows), so that no stride of one tensor stands in for
another's.
"""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity, oracle_full, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

LAYOUTS = ["bshd", "packed_qkv", "kv_broadcast", "padded", "mixed"]


def _strided(layout, q, k, v):
    """Device views of contiguous CPU (B, H, S, D) q, k, v in `layout`, and
    the contiguous CPU tensors they hold (equal to q, k, v except that
    kv_broadcast repeats head 0 of k and v over every head)."""
    B, H, S, D = q.shape
    if layout == "bshd":
        views = []
        for x in (q, k, v):
            buf = x.transpose(1, 2).contiguous().to(DEV)  # (B, S, H, D)
            views.append(buf.transpose(1, 2))
        return views, (q, k, v)
    if layout == "packed_qkv":
        buf = torch.stack([x.transpose(1, 2) for x in (q, k, v)], dim=2).contiguous().to(DEV)
        return [t.transpose(1, 2) for t in buf.unbind(dim=2)], (q, k, v)
    if layout == "kv_broadcast":
        k0, v0 = k[:, :1].expand(B, H, S, D), v[:, :1].expand(B, H, S, D)
        return ([q.to(DEV), k[:, :1].to(DEV).expand(B, H, S, D), v[:, :1].to(DEV).expand(B, H, S, D)],
                (q, k0.contiguous(), v0.contiguous()))
    if layout == "padded":
        views = []
        for x in (q, k, v):
            buf = torch.full((B, H, S, D + 64), float("nan"), dtype=x.dtype)
            buf[..., :D] = x
            views.append(buf.to(DEV)[..., :D])
        return views, (q, k, v)
    if layout == "mixed":
        q_view = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)  # rows H * D apart
        views = [q_view]
        for x in (k, v):  # rows D + 64 apart
            buf = torch.full((B, H, S, D + 64), float("nan"), dtype=x.dtype)
            buf[..., :D] = x
            views.append(buf.to(DEV)[..., :D])
        return views, (q, k, v)
    raise ValueError(layout)


def _out_like(layout, B, H, S, D, dtype):
    """o for the layout: a (B, S, H, D) buffer's view for the projection-style
    layouts, rows padded with NaN for `padded`, else contiguous."""
    if layout in ("bshd", "packed_qkv"):
        return torch.empty((B, S, H, D), dtype=dtype, device=DEV).transpose(1, 2)
    if layout == "padded":
        return torch.full((B, H, S, D + 64), float("nan"), dtype=dtype, device=DEV)[..., :D]
    return None


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_strided_equals_contiguous_bitwise(layout, D, dtype):
    for causal in (False, True):
        B, H, S = 2, 3, 200
        announce(f"strided {layout} D={D} {dtype} causal={causal}")
        w = wl.Workload("strided", B, H, S, D, dtype, causal)
        q, k, v = wl.make_qkv(w, seed=D + S)
        views, (qc, kc, vc) = _strided(layout, q, k, v)
        assert not all(t.is_contiguous() for t in views)
        o_s, lse_s = fa.attention(*views, causal=causal, scale=w.scale,
                                  out=_out_like(layout, B, H, S, D, q.dtype))
        o_c, lse_c = fa.attention(qc.to(DEV), kc.to(DEV), vc.to(DEV), causal=causal,
                                  scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_c), f"{layout}: O differs from the contiguous call"
        assert torch.equal(lse_s, lse_c), f"{layout}: lse differs from the contiguous call"


@pytest.mark.parametrize("layout,D,dtype,causal,S", [
    ("packed_qkv", 128, "f16", True, 333),
    ("packed_qkv", 64, "bf16", False, 257),
    ("bshd", 256, "bf16", True, 130),
    ("kv_broadcast", 128, "f16", True, 300),
    ("padded", 64, "f16", False, 129),
    ("mixed", 256, "f16", True, 161),
])
def test_strided_parity_with_oracle(layout, D, dtype, causal, S):
    B, H = 2, 3
    what = f"strided oracle {layout} D={D} {dtype} causal={causal} S={S}"
    announce(what)
    w = wl.Workload("strided", B, H, S, D, dtype, causal)
    q, k, v = wl.make_qkv(w, seed=7)
    views, (qc, kc, vc) = _strided(layout, q, k, v)
    o, lse = fa.attention(*views, causal=causal, scale=w.scale,
                          out=_out_like(layout, B, H, S, D, q.dtype))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(qc, kc, vc, causal, w.scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, what)


def test_strided_writes_only_os_rows():
    """Padding between o's rows keeps its NaN bytes; lse's neighbours too."""
    B, H, S, D = 2, 4, 190, 128
    announce("strided padding untouched")
    w = wl.Workload("strided", B, H, S, D, "f16", True)
    q, k, v = wl.make_qkv(w, seed=11)
    views, _ = _strided("padded", q, k, v)
    buf = torch.full((B, H, S, D + 64), float("nan"), dtype=q.dtype, device=DEV)
    lse_buf = torch.full((B * H * S + 64,), 123.0, dtype=torch.float32, device=DEV)
    lse = lse_buf[32:32 + B * H * S].view(B, H, S)
    o, _ = fa.attention(*views, causal=True, scale=w.scale, out=buf[..., :D], lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    assert torch.isnan(buf[..., D:]).all()
    assert (lse_buf[:32] == 123.0).all() and (lse_buf[32 + B * H * S:] == 123.0).all()


def test_strided_layer_shape_packed_qkv():
    """The layer shape B=1, H=32, T=2048, D=128 from one packed QKV buffer:
    bitwise equal to the contiguous call, and sampled rows against the
    oracle."""
    B, H, S, D = 1, 32, 2048, 128
    announce("strided packed qkv B=1 H=32 T=2048 D=128")
    w = wl.Workload("strided", B, H, S, D, "f16", True)
    q, k, v = wl.make_qkv(w, seed=0)
    views, _ = _strided("packed_qkv", q, k, v)
    o_s, lse_s = fa.attention(*views, causal=True, scale=w.scale,
                              out=_out_like("packed_qkv", B, H, S, D, q.dtype))
    o_c, lse_c = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(lse_s, lse_c)
    rows = sample_rows(B, H, S, seed=3)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, True, w.scale)
    o_rows = o_s.contiguous().reshape(-1, D).cpu()[torch.from_numpy(rows)]
    lse_rows = lse_s.reshape(-1).cpu()[torch.from_numpy(rows)]
    assert_parity(o_rows, lse_rows, o_ref, lse_ref, "f16", "packed qkv layer shape")


def test_strided_rejects_bad_strides():
    B, H, S, D = 1, 2, 64, 64
    q = torch.zeros((B, S, H, D + 4), dtype=torch.float16, device=DEV)[..., :D].transpose(1, 2)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(q, q, q)  # row stride H * (D + 4): not 16-byte aligned rows
    assert e.value.status == fa.FA2_ERR_STRIDE
    x = torch.zeros((B, H, S, D), dtype=torch.float16, device=DEV)
    bad_out = torch.empty((B, S, D), dtype=torch.float16, device=DEV).unsqueeze(1).expand(B, H, S, D)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(x, x, x, out=bad_out)  # every head's O in the same rows
    assert e.value.status == fa.FA2_ERR_STRIDE


def test_strided_d64_long_sequence_tile():
    """The D = 64 long-sequence tile (S >= 8192) on packed QKV views: bitwise
    equal to the contiguous call."""
    B, H, S, D = 1, 2, 8200, 64
    announce("strided packed qkv d64 S=8200")
    w = wl.Workload("strided", B, H, S, D, "bf16", True)
    q, k, v = wl.make_qkv(w, seed=5)
    views, _ = _strided("packed_qkv", q, k, v)
    o_s, lse_s = fa.attention(*views, causal=True, scale=w.scale,
                              out=_out_like("packed_qkv", B, H, S, D, q.dtype))
    o_c, lse_c = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(lse_s, lse_c)


@pytest.mark.parametrize("layout", ["packed_qkv", "mixed"])
def test_strided_multi_round_grid(layout):
    """A grid of three workgroups per compute unit (768 query tiles), whose
    last quarter takes tickets: strided views bitwise equal to the
    contiguous call, and sampled rows against the oracle."""
    B, H, S, D = 1, 12, 8192, 128
    announce(f"strided multi-round {layout} B={B} H={H} S={S}")
    w = wl.Workload("strided", B, H, S, D, "f16", True)
    q, k, v = wl.make_qkv(w, seed=13)
    views, _ = _strided(layout, q, k, v)
    o_s, lse_s = fa.attention(*views, causal=True, scale=w.scale, balanced=False,
                              out=_out_like(layout, B, H, S, D, q.dtype))
    o_c, lse_c = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=w.scale,
                              balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(lse_s, lse_c)
    rows = sample_rows(B, H, S, seed=4)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, True, w.scale)
    o_rows = o_s.contiguous().reshape(-1, D).cpu()[torch.from_numpy(rows)]
    lse_rows = lse_s.reshape(-1).cpu()[torch.from_numpy(rows)]
    assert_parity(o_rows, lse_rows, o_ref, lse_ref, "f16", f"strided multi-round {layout}")
