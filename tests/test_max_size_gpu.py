"""Long single heads near the size limits of the boundary, against the fp64
oracle on sampled rows.

fa2_fwd addresses one head of K or V with 32-bit byte offsets and accepts
(S + 256) * D * 2 bytes up to 2^31 - 1 per head. These cases put a head of
K and V at 256 MiB (S = 2^20 + 3, D = 128) and at 1 GiB (S = 2^21 + 5,
D = 256), so that tile offsets pass 2^28 and 2^30 bytes, the key loop runs
16K-64K tiles, and the last tile is ragged. Rows are compared at the
parity bar: max |O - O_ref| <= 2e-3 (fp16) / 1.6e-2 (bf16), lse relative
error <= 1e-4.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import announce, assert_parity, oracle_rows, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

CASES = [
    wl.Workload("long_head_s1048579_d128", 1, 1, (1 << 20) + 3, 128, "f16", False),
    wl.Workload("long_head_s2097157_d256", 1, 1, (1 << 21) + 5, 256, "bf16", True),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_long_head_sampled(w):
    # inside the boundary's limit on one head's bytes
    assert (w.S + 256) * w.D * 2 <= 2**31 - 1
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
