"""fa2_fwd_balanced: the key split of small grids.

When a launch has too few query tiles to keep the GPU busy to its end, the
keys of each tile are cut into chunks that run as separate workgroups and a
second kernel merges the chunks' (O~, m, l). The merge is exact algebra
(the rescaling of the guide's delayed-rescale recurrence, across chunks), so
the result must meet the same parity bar against the fp64 oracle as the
unsplit launch, on every row: the rows of one-chunk tiles (below row0,
written by the prefill kernel) and of split tiles (written by the merge).
Shapes that do not split must give fa2_fwd's result bit for bit.
"""
import numpy as np
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity, oracle_full, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

# (B, H, S): these split on a 256-CU MI355X at every head dim, causal or
# not (1 to 6 chunks per tile; S = 2049 leaves a one-row last tile);
# (1, 2, 600), (1, 1, 1) and (1, 2, 256) run unsplit.
SPLIT = [(1, 2, 2048), (2, 1, 1500), (1, 3, 2049), (1, 1, 3000)]
UNSPLIT = [(1, 2, 600), (1, 1, 1), (1, 2, 256)]


def _run(q, k, v, causal, scale, balanced=True, workspace=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale, balanced=balanced,
                          workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_split_matches_oracle(D, dtype, causal):
    for B, H, S in SPLIT:
        what = f"balanced D={D} {dtype} causal={causal} B={B} H={H} S={S}"
        announce(what)
        assert fa.fa2_fwd_balanced_workspace_bytes(B, H, S, D, int(causal)) > 0, \
            f"{what}: expected a key split"
        w = wl.Workload("bal", B, H, S, D, dtype, causal)
        q, k, v = wl.make_qkv(w, seed=S + D)
        o, lse = _run(q, k, v, causal, w.scale)
        o_ref, lse_ref = oracle_full(q, k, v, causal, w.scale)
        assert_parity(o, lse, o_ref, lse_ref, dtype, what)
        # the unsplit launch on the same inputs meets the same bar
        o1, lse1 = _run(q, k, v, causal, w.scale, balanced=False)
        assert_parity(o1, lse1, o_ref, lse_ref, dtype, what + " (unsplit)")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_split_negative_scale(D):
    """The key split with scale = -1/sqrt(D): each chunk's first-tile max is
    taken in the scaled domain, so the merged rows meet the bar too."""
    for causal in (True, False):
        B, H, S = SPLIT[0]
        what = f"balanced negative scale D={D} causal={causal} B={B} H={H} S={S}"
        announce(what)
        w = wl.Workload("bal", B, H, S, D, "f16", causal)
        q, k, v = wl.make_qkv(w, seed=S + D + 1)
        o, lse = _run(q, k, v, causal, -w.scale)
        o_ref, lse_ref = oracle_full(q, k, v, causal, -w.scale)
        assert_parity(o, lse, o_ref, lse_ref, "f16", what)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_unsplit_shapes_equal_fa2_fwd(D, causal):
    for B, H, S in UNSPLIT:
        announce(f"balanced unsplit D={D} causal={causal} B={B} H={H} S={S}")
        assert fa.fa2_fwd_balanced_workspace_bytes(B, H, S, D, int(causal)) == 0
        w = wl.Workload("bal", B, H, S, D, "f16", causal)
        q, k, v = wl.make_qkv(w, seed=S)
        o, lse = _run(q, k, v, causal, w.scale)
        o1, lse1 = _run(q, k, v, causal, w.scale, balanced=False)
        assert torch.equal(o, o1) and torch.equal(lse, lse1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_peaky_rows(dtype):
    """Q and K x3 (logit std about 9): near one-hot rows whose maximum sits
    in one chunk, so the other chunks' weights 2^(m_g - M) are tiny."""
    for causal in (False, True):
        w = wl.Workload("bal_peaky", 1, 2, 3000, 128, dtype, causal, qk_mult=3.0)
        announce(f"balanced peaky {dtype} causal={causal}")
        assert fa.fa2_fwd_balanced_workspace_bytes(1, 2, 3000, 128, int(causal)) > 0
        q, k, v = wl.make_qkv(w, seed=11)
        o, lse = _run(q, k, v, causal, w.scale)
        o_ref, lse_ref = oracle_full(q, k, v, causal, w.scale)
        assert_parity(o, lse, o_ref, lse_ref, dtype, f"balanced peaky causal={causal}")


def test_split_is_deterministic_and_strided_equal():
    """Two calls give the same bits, and (B, S, H, D) views of the same
    values give the contiguous call's bits (the plan does not depend on
    strides)."""
    w = wl.Workload("bal", 2, 1, 1500, 128, "bf16", True)
    announce("balanced determinism and strides")
    q, k, v = (x.to(DEV) for x in wl.make_qkv(w, seed=5))
    o_a, l_a = fa.attention(q, k, v, causal=True)
    o_b, l_b = fa.attention(q, k, v, causal=True)
    qs, ks_, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    obuf = torch.full((2, 1500, 1, 128 + 64), float("nan"), dtype=q.dtype, device=DEV)
    o_s, l_s = fa.attention(qs, ks_, vs, causal=True, out=obuf[..., :128].transpose(1, 2))
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    assert torch.equal(o_s, o_a) and torch.equal(l_s, l_a)
    assert torch.isnan(obuf[..., 128:]).all()


@pytest.mark.parametrize("w", [wl.ONE_GPU_SHARE,
                               wl.Workload("share_b1_h4_s8192_d256", 1, 4, 8192, 256, "bf16", True)],
                         ids=lambda w: w.name)
def test_split_full_size_rows(w):
    """The benchmark shapes that split, at full size: sampled rows, and the
    rows on both sides of every multiple of 128 (the query tile height) in
    the first and last heads, which include row0 (the first merged row) and
    every chunk boundary (chunks are whole query tiles' worth of keys)."""
    need = fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, int(w.causal))
    announce(f"balanced full size {w.name} workspace {need}")
    assert need > 0
    q, k, v = wl.make_qkv(w, seed=3)
    o, lse = _run(q, k, v, w.causal, w.scale)
    rows = set(sample_rows(w.B, w.H, w.S, seed=3).tolist())
    for r in range(128, w.S, 128):
        for i in (r - 1, r):
            rows.update({i, (w.B * w.H - 1) * w.S + i})
    rows = np.array(sorted(rows), dtype=np.int64)
    o_ref, lse_ref = oracle_rows(q, k, v, rows, w.causal, w.scale)
    o_s = o.reshape(-1, w.D)[torch.from_numpy(rows)]
    lse_s = lse.reshape(-1)[torch.from_numpy(rows)]
    assert_parity(o_s, lse_s, o_ref, lse_ref, w.dtype, f"{w.name} balanced ({len(rows)} rows)")


def test_workspace_errors():
    B, H, S, D = 1, 2, 2048, 128
    need = fa.fa2_fwd_balanced_workspace_bytes(B, H, S, D, 1)
    assert need > 0
    q = torch.zeros((B, H, S, D), dtype=torch.float16, device=DEV)
    k, v, o = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros((B, H, S), dtype=torch.float32, device=DEV)
    ws = torch.zeros((need + 256,), dtype=torch.uint8, device=DEV)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D,
            None, 1, 0.1, fa.FA2_F16)
    s = torch.cuda.current_stream().cuda_stream
    assert fa.fa2_fwd_balanced(*args, None, need, s) == fa.FA2_ERR_WORKSPACE
    assert fa.fa2_fwd_balanced(*args, ws.data_ptr(), need - 1, s) == fa.FA2_ERR_WORKSPACE
    assert fa.fa2_fwd_balanced(*args, ws.data_ptr() + 8, need, s) == fa.FA2_ERR_WORKSPACE
    # a workspace over o
    big = torch.zeros((max(need, o.numel() * 2) + 256,), dtype=torch.uint8, device=DEV)
    o_in = big[:o.numel() * 2].view(torch.float16)
    assert fa.fa2_fwd_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_in.data_ptr(),
                               lse.data_ptr(), B, H, S, D, None, 1, 0.1, fa.FA2_F16,
                               big.data_ptr(), need, s) == fa.FA2_ERR_ALIAS
    assert fa.fa2_fwd_balanced(*args, ws.data_ptr(), need, s) == fa.FA2_OK
    # a shape that does not split takes no workspace
    assert fa.fa2_fwd_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), 1, 1, 1, D, None, 1, 0.1, fa.FA2_F16, None, 0,
                               s) == fa.FA2_OK
    torch.cuda.synchronize()
