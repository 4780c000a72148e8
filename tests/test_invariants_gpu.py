"""Properties of the HIP path that hold at any size: exact special cases,
determinism, untouched memory around the outputs, streams and error paths."""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu


def _inputs(B, H, S, D, dtype, seed=0):
    w = wl.Workload("inv", B, H, S, D, dtype, True)
    q, k, v = wl.make_qkv(w, seed)
    return w, q.to(DEV), k.to(DEV), v.to(DEV)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_row0_is_v0_bit_exact(D, dtype):
    """Causal row 0 attends to key 0 only: P = 2^0 = 1, l = 1, so O[0] = V[0]
    exactly and lse[0] = scale q0.k0."""
    announce(f"row0 D={D} {dtype}")
    w, q, k, v = _inputs(2, 3, 1000, D, dtype, seed=1)
    o, lse = fa.attention(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    ref = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) * w.scale
    assert torch.allclose(lse[:, :, 0].double(), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_v_ones_gives_ones(D, dtype, causal):
    announce(f"v=1 D={D} {dtype} causal={causal}")
    w, q, k, v = _inputs(1, 2, 777, D, dtype, seed=2)
    v = torch.ones_like(v)
    o, _ = fa.attention(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    # sum_j P_j * 1 / l: P is rounded before the product while l sums the
    # unrounded P, so O is 1 within the rounding of P (a few ulps of fp32)
    # and then rounded once to the output dtype.
    ulp = 2.0 ** -10 if dtype == "f16" else 2.0 ** -7
    assert (o.double() - 1.0).abs().max().item() <= ulp


@pytest.mark.parametrize("causal", [False, True])
def test_deterministic(causal):
    """No atomics and a fixed reduction order: two runs are bitwise equal."""
    announce(f"determinism causal={causal}")
    w, q, k, v = _inputs(2, 4, 1500, 128, "f16", seed=3)
    o1, l1 = fa.attention(q, k, v, causal=causal, scale=w.scale)
    o2, l2 = fa.attention(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_outputs_leave_neighbours_untouched(D):
    """o and lse are carved out of larger sentinel-filled buffers; nothing
    outside (B, H, S, D) / (B, H, S) is written (tail rows beyond S included)."""
    announce(f"guard D={D}")
    w, q, k, v = _inputs(2, 2, 333, D, "bf16", seed=4)
    n = q.numel()
    nl = 2 * 2 * 333
    g = 4096
    obuf = torch.full((g + n + g,), 7.0, dtype=q.dtype, device=DEV)
    lbuf = torch.full((g + nl + g,), -3.0, dtype=torch.float32, device=DEV)
    o = obuf[g:g + n].view(q.shape)
    lse = lbuf[g:g + nl].view(2, 2, 333)
    fa.attention(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:g] == 7.0).all() and (obuf[g + n:] == 7.0).all()
    assert (lbuf[:g] == -3.0).all() and (lbuf[g + nl:] == -3.0).all()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_kv_permutation_invariance():
    announce("kv permutation")
    w, q, k, v = _inputs(1, 2, 640, 128, "f16", seed=5)
    perm = torch.randperm(640, generator=torch.Generator().manual_seed(0)).to(DEV)
    o1, l1 = fa.attention(q, k, v, causal=False, scale=w.scale)
    o2, l2 = fa.attention(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(),
                          causal=False, scale=w.scale)
    torch.cuda.synchronize()
    assert (o1.double() - o2.double()).abs().max().item() <= 2e-3
    assert ((l1 - l2).abs() / l1.abs().clamp_min(1)).max().item() <= 1e-5


def test_side_stream():
    """The launch goes to the stream it is given and does not synchronise."""
    announce("side stream")
    w, q, k, v = _inputs(1, 4, 900, 64, "f16", seed=6)
    ref_o, ref_l = fa.attention(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, causal=True, scale=w.scale)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_explicit_stream_allocations():
    """attention() and attention_splitkv() given a stream other than the
    current one, on shapes whose partials go to a workspace the binding
    allocates: that workspace (and O, lse) must come from the launch
    stream's memory, so that allocations on the current stream made right
    after the call cannot reuse it while the kernels still run. The launch
    stream is kept busy first, the current stream then allocates and
    overwrites blocks of the workspace's size throughout, and the results
    must still match the oracle."""
    import oracle

    announce("explicit stream with a binding-allocated workspace")
    s = torch.cuda.Stream()
    busy = torch.randn(4096, 4096, device=DEV)
    cases = []
    # prefill with a key split (B=1, H=2, S=2048, D=128 causal splits)
    w = wl.Workload("bal", 1, 2, 2048, 128, "f16", True)
    assert fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, 1) > 0
    q, k, v = wl.make_qkv(w, seed=21)
    cases.append(("prefill", w, q, k, v))
    dw = wl.DecodeWorkload("dec", 1, 4, 16, 4096, 128, "f16", True)
    dq, dk, dv = wl.make_qkv_decode(dw, seed=22)
    cases.append(("splitkv", dw, dq, dk, dv))
    for kind, w, q, k, v in cases:
        qd, kd, vd = (x.to(DEV) for x in (q, k, v))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(8):
                busy = busy @ busy
                busy /= busy.abs().max()
        if kind == "prefill":
            need = fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, 1)
            o, lse = fa.attention(qd, kd, vd, causal=True, scale=w.scale, stream=s)
        else:
            n = fa.fa2_splitkv_splits(w.B, w.H, w.Sq, w.Sk)
            need = fa.fa2_splitkv_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, n)
            o, lse = fa.attention_splitkv(qd, kd, vd, causal=True, scale=w.scale, stream=s)
        # the current stream allocates and scribbles while the launch stream works
        for _ in range(64):
            junk = torch.empty((need,), dtype=torch.uint8, device=DEV)
            junk.fill_(0x7F)
            del junk
        s.synchronize()
        torch.cuda.synchronize()
        if kind == "prefill":
            o_ref, lse_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(),
                                                  v.double().numpy(), True, w.scale)
        else:
            o_ref, lse_ref = oracle.attention_kv_f64(q.double().numpy(), k.double().numpy(),
                                                     v.double().numpy(), True, w.scale)
        assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, "f16", f"{kind} on a side stream")


def test_unsupported_inputs_fail_loudly():
    announce("error paths")
    x = torch.zeros(1, 1, 64, 96, dtype=torch.float16, device=DEV)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(x, x, x)
    assert e.value.status == fa.FA2_ERR_HEADDIM
    y = torch.zeros(1, 1, 64, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(y, y, y)
    assert e.value.status == fa.FA2_ERR_DTYPE
    z = torch.zeros(1, 1, 64, 64, dtype=torch.float16, device=DEV)
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(z, z, z, scale=float("nan"))
    assert e.value.status == fa.FA2_ERR_SCALE
    with pytest.raises(fa.FA2Error) as e:
        fa.attention(z, z, z, out=z)  # o aliases q
    assert e.value.status == fa.FA2_ERR_ALIAS
