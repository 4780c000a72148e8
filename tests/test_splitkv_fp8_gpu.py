"""Split-KV attention against an FP8 (e4m3) KV cache: fa2_fwd_splitkv_fp8.

The codes convert exactly to the matrix cores' 16-bit type on the GPU, so
the path computes fa2_fwd_splitkv's arithmetic on the dequantized K and V:
- with power-of-two descales every rescaling is exact, and the result must
  agree with fa2_fwd_splitkv on the dequantized values (held exactly in fp16
  and bf16) to within a few units in the last place of O and 1e-5 in lse:
  the only difference is the order in which q . k sums its fp32 partial
  products (the FP8 path groups head dims 32 u + 16 hi + 8 v .. + 7 per
  k-step), which can flip the rounding of a P or of an output;
- with any descales, the result meets the parity bar against the fp64
  oracle evaluated on the dequantized values (codes * descale, exact in
  fp64).
"""
import pytest
import torch

import flashattention_tiled_amd as fa
import oracle
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu

CASES = [(1, 1), (1, 33), (1, 1000), (16, 777), (33, 100), (70, 300), (5, 2)]


def _w(Sq, Sk, D, dtype, causal, kd, vd):
    return wl.DecodeWorkload("kv8", 2, 2, Sq, Sk, D, dtype, causal, kv="e4m3", k_descale=kd,
                             v_descale=vd)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_matches_16bit_path(D, dtype):
    for Sq, Sk in CASES:
        for causal in (False, True):
            if causal and Sq > Sk:
                continue
            w = _w(Sq, Sk, D, dtype, causal, 2.0 ** -6, 2.0 ** -5)
            announce(f"kv8 vs 16-bit D={D} {dtype} Sq={Sq} Sk={Sk} causal={causal}")
            q, k8, v8 = wl.make_qkv_decode_fp8(w, seed=Sq * 1000 + Sk)
            kq = wl.dequantize_fp8(k8, w.k_descale).to(w.torch_dtype)
            vq = wl.dequantize_fp8(v8, w.v_descale).to(w.torch_dtype)
            # the dequantized values are exact in the 16-bit type
            assert torch.equal(kq.double(), wl.dequantize_fp8(k8, w.k_descale))
            qd = q.to(DEV)
            o8, l8 = fa.attention_splitkv(qd, k8.to(DEV), v8.to(DEV), causal=causal,
                                          scale=w.scale, n_split=3, k_descale=w.k_descale,
                                          v_descale=w.v_descale)
            o16, l16 = fa.attention_splitkv(qd, kq.to(DEV), vq.to(DEV), causal=causal,
                                            scale=w.scale, n_split=3)
            torch.cuda.synchronize()
            ulp = 4 * (2.0 ** -10 if dtype == "f16" else 2.0 ** -7)  # four output ulps
            o8d, o16d = o8.double(), o16.double()
            d_o = ((o8d - o16d).abs() / o16d.abs().clamp(min=1.0)).max().item()
            d_l = ((l8.double() - l16.double()).abs() / l16.double().abs().clamp(min=1.0)).max().item()
            print(f"[kv8 vs 16-bit] rel |dO| {d_o:.3e} (bound {ulp:.1e}), lse {d_l:.3e}", flush=True)
            assert d_o <= ulp, f"O differs from the 16-bit path by {d_o:.3e}"
            assert d_l <= 1e-5, f"lse differs from the 16-bit path by {d_l:.3e}"


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_parity_with_oracle(D, dtype):
    for Sq, Sk in CASES:
        for causal in (False, True):
            if causal and Sq > Sk:
                continue
            for n_split in (1, 0, 64):
                w = _w(Sq, Sk, D, dtype, causal, 0.0123, 0.0371)
                what = f"kv8 oracle D={D} {dtype} Sq={Sq} Sk={Sk} causal={causal} n_split={n_split}"
                announce(what)
                q, k8, v8 = wl.make_qkv_decode_fp8(w, seed=Sq + 7 * Sk)
                o, lse = fa.attention_splitkv(q.to(DEV), k8.to(DEV), v8.to(DEV), causal=causal,
                                              scale=w.scale, n_split=n_split,
                                              k_descale=w.k_descale, v_descale=w.v_descale)
                torch.cuda.synchronize()
                o_ref, lse_ref = oracle.attention_kv_f64(
                    q.double().numpy(), wl.dequantize_fp8(k8, w.k_descale).numpy(),
                    wl.dequantize_fp8(v8, w.v_descale).numpy(), causal, w.scale)
                assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, what)


@pytest.mark.parametrize("w", wl.DECODE_FP8, ids=lambda w: w.name)
def test_fp8_decode_shapes(w):
    """The benchmark decoding shapes against an FP8 cache, every output."""
    announce(f"kv8 {w.name}")
    q, k8, v8 = wl.make_qkv_decode_fp8(w, seed=0)
    o, lse = fa.attention_splitkv(q.to(DEV), k8.to(DEV), v8.to(DEV), causal=w.causal,
                                  scale=w.scale, k_descale=w.k_descale, v_descale=w.v_descale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_kv_f64(q.double().numpy(),
                                             wl.dequantize_fp8(k8, w.k_descale).numpy(),
                                             wl.dequantize_fp8(v8, w.v_descale).numpy(),
                                             w.causal, w.scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, w.dtype, w.name)


def test_fp8_rejects_bad_descales():
    q = torch.zeros((1, 1, 1, 64), dtype=torch.float16, device=DEV)
    k = torch.zeros((1, 1, 64, 64), dtype=torch.float8_e4m3fn, device=DEV)
    for kd, vd in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        with pytest.raises(fa.FA2Error) as e:
            fa.attention_splitkv(q, k, k, k_descale=kd, v_descale=vd)
        assert e.value.status == fa.FA2_ERR_SCALE
