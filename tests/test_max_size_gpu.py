"""Long single heads and heads past 2 GiB, against the fp64 oracle.

The kernels address each K or V tile from a 64-bit start and its rows with
32-bit offsets from there, so a head may span any size. These cases put a
head of K and V at 256 MiB (S = 2^20 + 3, D = 128) and at 1 GiB
(S = 2^21 + 5, D = 256), so that the key loop runs 16K-64K tiles and the
last tile is ragged, and past 2 GiB: a strided prefill whose K and V rows
are 4 MiB apart (a 2.3 GiB head) and a decode against 2^23 + 5 cached keys
(K and V 2 GiB each). Rows are compared at the parity bar: max
|O - O_ref| <= 2e-3 (fp16) / 1.6e-2 (bf16), lse relative error <= 1e-4.
"""
import numpy as np
import pytest
import torch

import workloads as wl
import flashattention_tiled_amd as fa
import oracle
from gpu_helpers import DEV, announce, assert_parity, oracle_rows, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

CASES = [
    wl.Workload("long_head_s1048579_d128", 1, 1, (1 << 20) + 3, 128, "f16", False),
    wl.Workload("long_head_s2097157_d256", 1, 1, (1 << 21) + 5, 256, "bf16", True),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_long_head_sampled(w):
    announce(f"long head {w}")
    q, k, v = wl.make_qkv(w, seed=11)
    o, lse = run_gpu(q, k, v, w.causal, w.scale)
    S = w.S
    rows = set(sample_rows(1, 1, S, n_random=16, seed=w.S).tolist())
    # both sides of the last tile boundaries and the last rows
    rows.update(i for i in (S - 257, S - 256, S - 129, S - 128, S - 127, S - 3) if i >= 0)
    rows = np.array(sorted(rows), dtype=np.int64)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, w.causal, w.scale)
    idx = torch.from_numpy(rows)
    assert_parity(o.reshape(-1, w.D)[idx], lse.reshape(-1)[idx], o_ref, lse_ref, w.dtype,
                  f"{w.name} ({len(rows)} rows)")


def test_strided_prefill_head_past_2gib():
    """K and V as column views of one (S, 2^21) fp16 buffer: rows 4 MiB
    apart, so the last rows of the head lie past 2^31 bytes from its start.
    Every output against the oracle on contiguous copies."""
    S, D, row = 600, 128, 1 << 21
    announce(f"strided prefill, head of {(S - 1) * row * 2 / 2**30:.2f} GiB")
    w = wl.Workload("strided_2gib", 1, 1, S, D, "f16", True)
    q, k, v = wl.make_qkv(w, seed=23)
    buf = torch.zeros((S, row), dtype=torch.float16, device=DEV)
    buf[:, :D] = k[0, 0].to(DEV)
    buf[:, D:2 * D] = v[0, 0].to(DEV)
    kd = buf[:, :D].unsqueeze(0).unsqueeze(0)
    vd = buf[:, D:2 * D].unsqueeze(0).unsqueeze(0)
    assert kd.stride(2) == row and (S - 1) * row * 2 > 2**31
    for causal in (True, False):
        o, lse = fa.attention(q.to(DEV), kd, vd, causal=causal, scale=w.scale, balanced=False)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_f64(q.double().numpy(), k.double().numpy(),
                                              v.double().numpy(), causal, w.scale)
        assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, "f16",
                      f"strided head past 2 GiB causal={causal}")
    del buf


def test_decode_head_past_2gib():
    """Three queries against 2^23 + 5 cached keys at D = 128 (K and V 2 GiB
    each): the split-KV chunks of the last keys start past 2^31 bytes.
    Every output against the oracle's KV form."""
    dw = wl.DecodeWorkload("decode_2gib", 1, 1, 3, (1 << 23) + 5, 128, "f16", True)
    announce(f"decode, head of {dw.Sk * dw.D * 2 / 2**30:.2f} GiB")
    q, k, v = wl.make_qkv_decode(dw, seed=29)
    o, lse = fa.attention_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=dw.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    o_ref, lse_ref = oracle.attention_kv_f64(q.double().numpy(), k.double().numpy(),
                                             v.double().numpy(), True, dw.scale)
    assert_parity(o, lse, o_ref, lse_ref, "f16", "decode head past 2 GiB")
