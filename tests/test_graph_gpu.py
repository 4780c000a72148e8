"""The entry points under HIP graph capture, through the C ABI.

Each call is captured once into a graph (torch.cuda.CUDAGraph) and the graph
is replayed three times. Before each replay new inputs are written in place
and the same call is made eagerly on them; every replay's O and lse must equal
the eager call's bit for bit (the kernels are deterministic), and the first
replay of each small case also meets the parity bar against the fp64 oracle.
The library records no memset and no allocation on the stream, so a captured
call is the same launches as an eager one.

Covered: fa2_fwd on the main tile and on the key-group tile, fa2_fwd_balanced
(the key split and its merge kernel, with a caller's workspace),
fa2_fwd_splitkv_noalloc (the split-KV call for callers that cannot allocate,
its partials in the library's own scratch) and fa2_fwd_fp8.
"""
import pytest
import torch

import flashattention_tiled_amd as fa
import oracle
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _code(dtype: str) -> int:
    return fa.FA2_F16 if dtype == "f16" else fa.FA2_BF16


def _replay_equals_eager(call, inputs, fresh, outs_g, outs_e, what):
    """Warm up, capture call(outs_g), then per replay: fresh inputs written in
    place, an eager call into outs_e, the replay; compare."""
    stream = torch.cuda.current_stream().cuda_stream
    assert call(*outs_e, stream) == fa.FA2_OK
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(graph):
        status.append(call(*outs_g, torch.cuda.current_stream().cuda_stream))
    assert status == [fa.FA2_OK], (what, status)
    for r in range(REPLAYS):
        for x, y in zip(inputs, fresh(r)):
            x.copy_(y)
        for t in outs_g:
            t.fill_(float("nan"))
        assert call(*outs_e, torch.cuda.current_stream().cuda_stream) == fa.FA2_OK
        graph.replay()
        torch.cuda.synchronize()
        for t_g, t_e in zip(outs_g, outs_e):
            assert torch.equal(t_g, t_e), f"{what}: replay {r} differs from the eager call"
    return graph


def _prefill_inputs(w, seed):
    q, k, v = wl.make_qkv(w, seed=seed)
    return q.to(DEV), k.to(DEV), v.to(DEV)


@pytest.mark.parametrize("B,H,S,dt,tile", [(1, 8, 1000, "f16", "main"),
                                           (1, 32, 2048, "bf16", "key groups")],
                         ids=["main-tile", "key-group-tile"])
def test_fa2_fwd_graph(B, H, S, dt, tile):
    w = wl.Workload(f"graph_{tile}", B, H, S, 128, dt, True)
    announce(f"graph capture fa2_fwd {tile} B={B} H={H} S={S} {dt}")
    q, k, v = _prefill_inputs(w, 1)
    outs_g = (torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device=DEV))
    outs_e = (torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device=DEV))

    def call(o, lse, stream):
        return fa.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, S, 128, 1, w.scale, _code(dt), stream)

    _replay_equals_eager(call, (q, k, v), lambda r: _prefill_inputs(w, 10 + r), outs_g, outs_e,
                         f"fa2_fwd {tile}")
    if S <= 1000:
        qc, kc, vc = (x.cpu() for x in (q, k, v))
        o_ref, lse_ref = oracle.attention_f64(qc.double().numpy(), kc.double().numpy(),
                                              vc.double().numpy(), True, w.scale)
        assert_parity(outs_g[0].cpu(), outs_g[1].cpu(), o_ref, lse_ref, dt,
                      f"graph fa2_fwd {tile}")


def test_fa2_fwd_balanced_graph():
    B, H, S, D = 1, 4, 8192, 128
    w = wl.Workload("graph_balanced", B, H, S, D, "f16", True)
    announce(f"graph capture fa2_fwd_balanced B={B} H={H} S={S}")
    need = fa.fa2_fwd_balanced_workspace_bytes(B, H, S, D, 1)
    assert need > 0, "the shape should take the key split"
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    q, k, v = _prefill_inputs(w, 2)
    outs_g = (torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device=DEV))
    outs_e = (torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device=DEV))

    def call(o, lse, stream):
        return fa.fa2_fwd_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, S, D, None, 1, w.scale, fa.FA2_F16,
                                   ws.data_ptr(), need, stream)

    _replay_equals_eager(call, (q, k, v), lambda r: _prefill_inputs(w, 20 + r), outs_g, outs_e,
                         "fa2_fwd_balanced")


def test_splitkv_noalloc_graph():
    dw = wl.DecodeWorkload("graph_decode", 2, 8, 3, 8192, 128, "bf16", True)
    announce(f"graph capture fa2_fwd_splitkv_noalloc {dw}")

    def fresh(r):
        q, k, v = wl.make_qkv_decode(dw, seed=30 + r)
        return q.to(DEV), k.to(DEV), v.to(DEV)

    q, k, v = fresh(-1)
    n_split = fa.fa2_splitkv_splits(dw.B, dw.H, dw.Sq, dw.Sk)
    shape_o = (dw.B, dw.H, dw.Sq, dw.D)
    outs_g = (torch.empty(shape_o, dtype=q.dtype, device=DEV),
              torch.empty((dw.B, dw.H, dw.Sq), dtype=torch.float32, device=DEV))
    outs_e = (torch.empty(shape_o, dtype=q.dtype, device=DEV),
              torch.empty((dw.B, dw.H, dw.Sq), dtype=torch.float32, device=DEV))

    def call(o, lse, stream):
        return fa.fa2_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), dw.B, dw.H, dw.Sq, dw.Sk, dw.D, 1,
                                          dw.scale, fa.FA2_BF16, n_split, stream)

    _replay_equals_eager(call, (q, k, v), fresh, outs_g, outs_e, "fa2_fwd_splitkv_noalloc")
    o_ref, lse_ref = oracle.attention_kv_f64(q.cpu().double().numpy(), k.cpu().double().numpy(),
                                             v.cpu().double().numpy(), True, dw.scale)
    assert_parity(outs_g[0].cpu(), outs_g[1].cpu(), o_ref, lse_ref, "bf16",
                  "graph fa2_fwd_splitkv_noalloc")


def test_fa2_fwd_fp8_graph():
    B, H, S, D = 1, 8, 1000, 128
    w = wl.Workload("graph_fp8", B, H, S, D, "f16", True)
    announce(f"graph capture fa2_fwd_fp8 B={B} H={H} S={S}")
    dq, dk, dv = wl.fp8_descales(w)

    def fresh(r):
        q, k, v = wl.make_qkv_fp8(w, seed=40 + r)
        return q.to(DEV), k.to(DEV), v.to(DEV)

    q, k, v = fresh(-1)
    outs_g = (torch.empty((B, H, S, D), dtype=torch.float16, device=DEV),
              torch.empty((B, H, S), dtype=torch.float32, device=DEV))
    outs_e = (torch.empty((B, H, S, D), dtype=torch.float16, device=DEV),
              torch.empty((B, H, S), dtype=torch.float32, device=DEV))

    def call(o, lse, stream):
        return fa.fa2_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, S, D, 1, w.scale, dq, dk, dv, fa.FA2_F16,
                              stream)

    _replay_equals_eager(call, (q, k, v), fresh, outs_g, outs_e, "fa2_fwd_fp8")
