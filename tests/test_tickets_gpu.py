"""The tickets of the prefill kernel's last workgroups, through the C ABI.

On grids of more than one round the last quarter of the workgroups take
their query tiles in the order they start, from a counter the library keeps
per (device, stream); a call being captured into a graph takes none and
keeps the fixed order. Every tile is computed the same way in either order,
so the results must be bit-identical to the captured call's:
- for several multi-round shapes, one after another on one stream (each
  launch must leave its counter at zero for the next, whatever its size);
- for two streams launching at once, each with its own counter, many times,
  and for hipStreamPerThread used by two host threads at once;
- for the FP8 prefill, which takes tickets from the same counters.
"""
import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu

# (B, H, S, D, dtype): every one more than 2 workgroups per compute unit on
# 256 units (a multi-round grid), so that the last quarter takes tickets
SHAPES = [
    (1, 12, 8192, 128, "f16"),    # 768 query tiles of 128 rows
    (2, 16, 2304, 256, "bf16"),   # 576, the unpipelined D = 256 tile
    (1, 40, 4000, 64, "f16"),     # 1280, D = 64
    (1, 12, 8192, 128, "f16"),    # the first again: its counter must be back at zero
]


def _inputs(B, H, S, D, dt, seed):
    w = wl.Workload("tickets", B, H, S, D, dt, True)
    q, k, v = (x.to(DEV) for x in wl.make_qkv(w, seed=seed))
    return w, q, k, v


def _call(w, q, k, v, o, lse, stream):
    code = fa.FA2_F16 if w.dtype == "f16" else fa.FA2_BF16
    return fa.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      w.B, w.H, w.S, w.D, 1, w.scale, code, stream)


def _fixed_order(w, q, k, v):
    """O and lse of a captured call (no tickets), from one graph replay."""
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=DEV)
    assert _call(w, q, k, v, o, lse, torch.cuda.current_stream().cuda_stream) == fa.FA2_OK
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(graph):
        status.append(_call(w, q, k, v, o, lse, torch.cuda.current_stream().cuda_stream))
    assert status == [fa.FA2_OK]
    o.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    return o.clone(), lse.clone()


def test_tickets_match_fixed_order_one_stream():
    for i, (B, H, S, D, dt) in enumerate(SHAPES):
        announce(f"tickets one stream B={B} H={H} S={S} D={D} {dt}")
        w, q, k, v = _inputs(B, H, S, D, dt, seed=50 + i)
        o_ref, lse_ref = _fixed_order(w, q, k, v)
        for rep in range(3):
            o = torch.full_like(q, float("nan"))
            lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
            assert _call(w, q, k, v, o, lse, torch.cuda.current_stream().cuda_stream) == fa.FA2_OK
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"{(B, H, S, D, dt)} call {rep}: O differs"
            assert torch.equal(lse, lse_ref), f"{(B, H, S, D, dt)} call {rep}: lse differs"


def test_tickets_two_streams_at_once():
    announce("tickets on two streams at once")
    w, q, k, v = _inputs(1, 12, 8192, 128, "f16", seed=60)
    w2, q2, k2, v2 = _inputs(1, 12, 8192, 128, "f16", seed=61)
    ref = _fixed_order(w, q, k, v)
    ref2 = _fixed_order(w2, q2, k2, v2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for _ in range(8):
        o, lse = torch.empty_like(q), torch.empty((1, 12, 8192), dtype=torch.float32, device=DEV)
        o2, lse2 = torch.empty_like(q2), torch.empty((1, 12, 8192), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()  # the outputs exist before either stream writes them
        assert _call(w, q, k, v, o, lse, s1.cuda_stream) == fa.FA2_OK
        assert _call(w2, q2, k2, v2, o2, lse2, s2.cuda_stream) == fa.FA2_OK
        outs.append((o, lse, o2, lse2))
    torch.cuda.synchronize()
    for i, (o, lse, o2, lse2) in enumerate(outs):
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"stream 1, round {i}"
        assert torch.equal(o2, ref2[0]) and torch.equal(lse2, ref2[1]), f"stream 2, round {i}"


def test_fp8_tickets_match_fixed_order():
    B, H, S, D = 1, 12, 8192, 128  # 768 query tiles
    announce(f"FP8 tickets B={B} H={H} S={S} D={D}")
    w = wl.Workload("tickets_fp8", B, H, S, D, "f16", True)
    q, k, v = (x.to(DEV) for x in wl.make_qkv_fp8(w, seed=70))
    dq, dk, dv = wl.fp8_descales(w)

    def call(o, lse, stream):
        return fa.fa2_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, S, D, 1, w.scale, dq, dk, dv, fa.FA2_F16, stream)

    o_ref = torch.empty((B, H, S, D), dtype=torch.float16, device=DEV)
    lse_ref = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    assert call(o_ref, lse_ref, torch.cuda.current_stream().cuda_stream) == fa.FA2_OK
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(graph):
        status.append(call(o_ref, lse_ref, torch.cuda.current_stream().cuda_stream))
    assert status == [fa.FA2_OK]
    o_ref.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    for rep in range(3):
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        assert call(o, lse, torch.cuda.current_stream().cuda_stream) == fa.FA2_OK
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"FP8 call {rep}: O differs from the fixed order"
        assert torch.equal(lse, lse_ref), f"FP8 call {rep}: lse differs from the fixed order"


def test_tickets_per_thread_default_streams():
    """hipStreamPerThread, one handle naming a different stream in each host
    thread: two threads launching on it at once get a counter each."""
    import threading

    per_thread = 2  # hipStreamPerThread
    announce("tickets on two threads' per-thread streams")
    w, q, k, v = _inputs(1, 12, 8192, 128, "f16", seed=80)
    w2, q2, k2, v2 = _inputs(1, 12, 8192, 128, "f16", seed=81)
    refs = [_fixed_order(w, q, k, v), _fixed_order(w2, q2, k2, v2)]
    jobs = [(w, q, k, v), (w2, q2, k2, v2)]
    outs = [[(torch.empty_like(q), torch.empty((1, 12, 8192), dtype=torch.float32, device=DEV))
             for _ in range(6)] for _ in range(2)]
    torch.cuda.synchronize()
    status = [[], []]

    def run(t):
        wt, qt, kt, vt = jobs[t]
        for o, lse in outs[t]:
            status[t].append(_call(wt, qt, kt, vt, o, lse, per_thread))
        # this thread's per-thread stream ends with the thread: wait for it here
        torch.cuda.synchronize()

    threads = [threading.Thread(target=run, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    for t in range(2):
        assert status[t] == [fa.FA2_OK] * 6, status[t]
        for i, (o, lse) in enumerate(outs[t]):
            assert torch.equal(o, refs[t][0]) and torch.equal(lse, refs[t][1]), f"thread {t}, call {i}"
