"""Split-KV attention on strided tensors (fa2_fwd_splitkv_strided): a KV
cache allocated for a maximum length and read up to the current one, a
(B, S, H, D) cache, and O written with padded rows. Only the addressing
differs from the contiguous call, so the results equal it bit for bit, for
16-bit and for FP8 K and V.
"""
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu


def _cache_view(x, layout, s_max):
    """x (B, H, Sk, D) on the GPU as a strided view: rows 0..Sk-1 of a
    (B, H, s_max, D) buffer ("max_len"), or of a (B, s_max, H, D) buffer
    ("bshd")."""
    B, H, Sk, D = x.shape
    # bytes through int views, which every element type supports
    it = torch.int16 if x.element_size() == 2 else torch.uint8
    xb = x.view(it).to(DEV)
    if layout == "max_len":
        buf = torch.zeros((B, H, s_max, D), dtype=it, device=DEV)
        buf[:, :, :Sk] = xb
        return buf.view(x.dtype)[:, :, :Sk]
    buf = torch.zeros((B, s_max, H, D), dtype=it, device=DEV)
    buf[:, :Sk] = xb.transpose(1, 2)
    return buf.view(x.dtype)[:, :Sk].transpose(1, 2)


@pytest.mark.parametrize("layout", ["max_len", "bshd"])
@pytest.mark.parametrize("kv8", [False, True])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_strided_cache_equals_contiguous(layout, kv8, D):
    for dtype in ("f16", "bf16"):
        for Sq, Sk, causal in ((1, 1000, True), (16, 777, True), (40, 300, False)):
            announce(f"splitkv strided {layout} kv8={kv8} D={D} {dtype} Sq={Sq} Sk={Sk}")
            w = wl.DecodeWorkload("skv", 2, 3, Sq, Sk, D, dtype, causal,
                                  kv="e4m3" if kv8 else "", k_descale=0.02, v_descale=0.03)
            q, k, v = (wl.make_qkv_decode_fp8 if kv8 else wl.make_qkv_decode)(w, seed=Sk + Sq)
            kw = dict(causal=causal, scale=w.scale, n_split=5, k_descale=w.k_descale,
                      v_descale=w.v_descale)
            # q from a (B, Sq, H, D) buffer, O into rows padded by 64 elements
            qs = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
            obuf = torch.full((2, 3, Sq, D + 64), float("nan"), dtype=q.dtype, device=DEV)
            o_s, l_s = fa.attention_splitkv(qs, _cache_view(k, layout, Sk + 37),
                                            _cache_view(v, layout, Sk + 37),
                                            out=obuf[..., :D], **kw)
            o_c, l_c = fa.attention_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
            torch.cuda.synchronize()
            assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c)
            assert torch.isnan(obuf[..., D:]).all()
