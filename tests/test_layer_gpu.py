"""FA2Attention, the attention layer around the kernel (the cookbook
notebook "FlashAttention-2 in an attention layer").

- Parity: the layer's output against the fp64 oracle's attention between
  the same projections, at a bound carried through the output projection.
- The notebook's own checks: output within 1e-3 of a reference layer whose
  attention is evaluated exactly (fp32, CPU; the notebook uses SDPA's math
  backend) with the same weights ("Numerical equivalence"), and peak memory
  growing no more than 5x when T grows 4x ("Memory growth").
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from flashattention_tiled_amd.layer import FA2Attention
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu


def _layer(d_model, heads, dtype=torch.float16, seed=0, frozen=True):
    torch.manual_seed(seed)
    layer = FA2Attention(d_model, heads).to(device=DEV, dtype=dtype)
    return layer.requires_grad_(not frozen)


def _input(B, T, d_model, dtype=torch.float16, seed=1):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn((B, T, d_model), generator=g, dtype=torch.float32).to(dtype).to(DEV)


@pytest.mark.parametrize("d_model,heads,T,dtype", [
    (1024, 16, 256, "f16"),   # the notebook's equivalence shape (D = 64)
    (1024, 8, 301, "bf16"),   # D = 128, ragged T
    (2048, 8, 200, "f16"),    # D = 256
])
def test_layer_parity_with_oracle(d_model, heads, T, dtype):
    """y = W_o attn(q, k, v) with (q, k, v) the layer's own QKV projection:
    the oracle evaluates attn in fp64 on those projections and W_o is applied
    in fp64. |y - y_ref| is bounded per output by sum_i |W_o[j, i]| * tol_O
    (the kernel's O tolerance) plus the rounding of y to the dtype."""
    B = 2
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    announce(f"layer oracle d={d_model} H={heads} T={T} {dtype}")
    layer = _layer(d_model, heads, tdt)
    x = _input(B, T, d_model, tdt)
    with torch.inference_mode():
        qkv = layer.qkv(x)
        y = layer.o(layer.attend(qkv))
    torch.cuda.synchronize()
    H, D = heads, d_model // heads
    qkv5 = qkv.view(B, T, 3, H, D).double().cpu()
    q, k, v = (qkv5[:, :, i].transpose(1, 2).contiguous().numpy() for i in range(3))
    o_ref, _ = oracle.attention_f64(q, k, v, True, 1.0 / np.sqrt(D))
    a_ref = np.ascontiguousarray(o_ref.transpose(0, 2, 1, 3)).reshape(B, T, d_model)
    w_o = layer.o.weight.double().cpu().numpy()  # (out, in)
    y_ref = a_ref @ w_o.T
    unit = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
    bound = np.abs(w_o).sum(axis=1) * wl.TOLERANCE_O[dtype] + 2 * unit * np.abs(y_ref) + 1e-6
    err = np.abs(y.double().cpu().numpy() - y_ref)
    print(f"[parity] layer: max|dy|={err.max():.3e}, worst err/bound {np.max(err / bound):.3f}")
    assert (err <= bound).all()


def test_layer_matches_exact_attention_within_1e_3():
    """The notebook's equivalence check at its shape: d_model 1024, 16 heads,
    T=256, fp16, the same weights, attention evaluated exactly (fp32 on the
    CPU) in the reference layer: max |y_fa2 - y_ref| < 1e-3."""
    announce("layer vs exact attention, notebook shape")
    d_model, heads, T = 1024, 16, 256
    layer = _layer(d_model, heads)
    x = _input(1, T, d_model)
    with torch.inference_mode():
        y = layer(x)
        qkv = layer.qkv(x).view(1, T, 3, heads, d_model // heads).float().cpu()
        q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
        attn = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        y_ref = layer.o(attn.transpose(1, 2).reshape(1, T, d_model).to(DEV, torch.float16))
    torch.cuda.synchronize()
    err = (y - y_ref).abs().max().item()
    print(f"[layer] max|y_fa2 - y_ref| = {err:.3e}")
    assert err < 1e-3


def _peak_mib(layer, T, d_model):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    x = _input(1, T, d_model)
    with torch.inference_mode():
        layer(x)
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() / 2 ** 20


def test_layer_memory_grows_linearly():
    """The notebook's memory check: T from 512 to 2048 (4x) grows the peak
    allocation at most 5x (the S x S scores are never stored)."""
    announce("layer memory growth")
    d_model, heads = 1024, 16
    layer = _layer(d_model, heads)
    small, large = _peak_mib(layer, 512, d_model), _peak_mib(layer, 2048, d_model)
    print(f"[layer] peak MiB: T=512 {small:.1f}, T=2048 {large:.1f}, growth {large / small:.2f}x")
    assert large / small <= 5.0


def test_layer_refuses_autograd():
    layer = _layer(1024, 16, frozen=False)
    x = _input(1, 64, 1024)
    with pytest.raises(RuntimeError):
        layer(x)
