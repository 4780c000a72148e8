"""fa2_fwd_splitkv_noalloc, the split-KV call that allocates nothing, through
the C ABI: on two calls in a row, the second on a smaller input, its O and
lse equal fa2_fwd_splitkv's on the same inputs and split count bit for bit
(the same kernels, with the partials in the library's scratch instead of a
workspace) and meet the parity bar against the fp64 oracle; a call whose
partials exceed the scratch is refused before any launch."""
import pytest
import torch

import flashattention_tiled_amd as fa
import oracle
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu


def _with_workspace(q, k, v, w, n_split):
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=DEV)
    need = fa.fa2_splitkv_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, n_split)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=DEV)
    st = fa.fa2_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr(), w.B, w.H, w.Sq, w.Sk, w.D, int(w.causal),
                            w.scale, fa.FA2_F16 if w.dtype == "f16" else fa.FA2_BF16, n_split,
                            ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA2_OK, fa.fa2_status_string(st)
    return o, lse


def _noalloc(q, k, v, w, n_split):
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.Sq), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.fa2_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), w.B, w.H, w.Sq, w.Sk, w.D, int(w.causal),
                                    w.scale, fa.FA2_F16 if w.dtype == "f16" else fa.FA2_BF16,
                                    n_split, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA2_OK, fa.fa2_status_string(st)
    return o, lse


@pytest.mark.parametrize("n_split", [0, 5])
def test_noalloc_matches_workspace_call(n_split):
    # a larger call first, then a smaller one that reuses the scratch's start
    shapes = [wl.DecodeWorkload("na_big", 4, 8, 40, 3000, 128, "bf16", True),
              wl.DecodeWorkload("na_small", 1, 2, 1, 500, 64, "f16", False)]
    for i, w in enumerate(shapes):
        what = f"noalloc call {i} {w} n_split={n_split}"
        announce(what)
        q, k, v = wl.make_qkv_decode(w, seed=31 + i)
        qd, kd, vd = (x.to(DEV) for x in (q, k, v))
        o1, l1 = _noalloc(qd, kd, vd, w, n_split)
        o2, l2 = _with_workspace(qd, kd, vd, w, n_split)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), what
        assert torch.equal(l1, l2), what
        o_ref, lse_ref = oracle.attention_kv_f64(q.double().numpy(), k.double().numpy(),
                                                 v.double().numpy(), w.causal, w.scale)
        assert_parity(o1.cpu(), l1.cpu(), o_ref, lse_ref, w.dtype, what)


def test_noalloc_refuses_oversized_call():
    announce("noalloc oversized")
    q = torch.zeros((8, 64, 64, 256), dtype=torch.float16, device=DEV)
    kv = torch.zeros((8, 64, 128, 256), dtype=torch.float16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((8, 64, 64), dtype=torch.float32, device=DEV)
    assert fa.fa2_splitkv_workspace_bytes(8, 64, 64, 128, 256, 4) > (16 << 20)
    st = fa.fa2_fwd_splitkv_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), 8, 64, 64, 128, 256, 0, 0.0625, fa.FA2_F16, 4,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA2_ERR_SCRATCH
