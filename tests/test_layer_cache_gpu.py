"""FA2Attention with a KV cache: a prompt, then single-token steps, then a
16-token chunk, with a 16-bit and with an FP8 (e4m3) cache.

Each step's attention output (the input of the output projection) is held
to the parity bar against the fp64 oracle evaluated on that step's queries
and on the cache as it stands after the step (for FP8, the codes times the
descales): the step's tokens are the last ones, causally aligned.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from flashattention_tiled_amd.layer import FA2Attention, KVCache
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu


def _values(cache):
    k, v = cache.view()
    if cache.fp8:
        return (wl.dequantize_fp8(k.cpu(), cache.k_descale).numpy(),
                wl.dequantize_fp8(v.cpu(), cache.v_descale).numpy())
    return k.double().cpu().numpy(), v.double().cpu().numpy()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_cached_steps_match_the_oracle(fp8, dtype):
    B, d_model, heads, max_len = 2, 1024, 8, 160
    D = d_model // heads
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    torch.manual_seed(0)
    layer = FA2Attention(d_model, heads).to(device=DEV, dtype=tdt).requires_grad_(False)
    cache = KVCache(B, heads, max_len, D, dtype=tdt, device=DEV, fp8=fp8, k_descale=1 / 48,
                    v_descale=1 / 40)
    g = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn((B, 122, d_model), generator=g).to(tdt).to(DEV)
    pos = 0
    for T in (100, 1, 1, 1, 1, 1, 16, 1):
        what = f"layer cache fp8={fp8} {dtype} step T={T} at {pos}"
        announce(what)
        with torch.inference_mode():
            qkv = layer.qkv(x[:, pos:pos + T])
            a = layer.attend_cached(qkv, cache)
        torch.cuda.synchronize()
        pos += T
        assert cache.length == pos
        q = qkv.view(B, T, 3, heads, D)[:, :, 0].transpose(1, 2).double().cpu().numpy()
        k, v = _values(cache)
        o_ref, lse_ref = oracle.attention_kv_f64(np.ascontiguousarray(q), k, v, True,
                                                 1.0 / np.sqrt(D))
        a_gpu = a.view(B, T, heads, D).transpose(1, 2).cpu()
        # lse is not returned by the layer: compare O alone (lse_ref against itself)
        assert_parity(a_gpu, torch.from_numpy(lse_ref).float(), o_ref, lse_ref, dtype, what)


def test_cache_overflow_raises():
    cache = KVCache(1, 2, 4, 64, device=DEV)
    k = torch.zeros((1, 2, 3, 64), dtype=torch.float16, device=DEV)
    cache.append(k, k)
    with pytest.raises(ValueError):
        cache.append(k, k)
