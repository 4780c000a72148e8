"""Per-workgroup timeline of the prefill kernel, a measurement aid.

`build` compiles the library's sources with -DFA2_TIMELINE into a library of
its own (libfa2_timeline.so beside libfa2.so, include/fa2_timeline.h), in which wave 0 of
every workgroup of a prefill launch records the 100 MHz real-time clock at
its start, after its prologue, after its key loop and at its end, with its
compute unit's hardware ids and its query tile. `run` launches fa2_fwd of
the named benchmark workloads on that library (after a warm-up of the
workload's own launches, which settles the clock), reads the stamps of one
launch and prints where its time went:

- the launch's span and the workgroups' average start (prologue), key-loop
  and end (epilogue) times;
- per XCD (XCC_ID): its workgroups' key-loop time per step and when its
  last workgroup ended;
- per compute unit: when its last workgroup ended, and the time from one
  workgroup's end to the next one's start on it;
- for launches of at least two workgroups per unit, the key-loop time per
  step of each unit's first and second resident workgroup of the first
  wave (launch order 0 .. n_cu - 1 and n_cu .. 2 n_cu - 1).

    python -m flashattention_tiled_amd.timeline build
    python -m flashattention_tiled_amd.timeline run [--workload NAME ...] [--warmup N]

The library's own build (libfa2.so) compiles the recording out: its kernels
are the ones timed here, without the stamps.
"""
from __future__ import annotations

import argparse
import collections
import ctypes
import os
import sys

import numpy as np

from .build import ROOT, TIMELINE_LIB_PATH, build_timeline

SLOTS = 8
TICK_US = 0.01  # s_memrealtime runs at 100 MHz


def summarize(words: np.ndarray, n_cu: int) -> dict:
    """Figures of one launch from its stamps: `words` is (n_wg, 8) uint64 in
    launch order, every row written (see include/fa2_timeline.h)."""
    b = words.astype(np.int64)
    n = b.shape[0]
    t0 = b[:, 0].min()
    t = [(b[:, j] - t0) * TICK_US for j in range(4)]
    hw = b[:, 4] & 0xFFFFFFFF
    xcc = (b[:, 4] >> 32) & 0xFF
    steps = np.maximum(b[:, 5] >> 32, 1)
    loop = t[2] - t[1]
    unit = xcc * 256 + ((hw >> 8) & 0xFF)  # XCC, then HW_ID's CU, SH and SE fields
    out = {
        "workgroups": n,
        "span_us": float(t[3].max()),
        "prologue_us": float((t[1] - t[0]).mean()),
        "loop_us_per_step": float((loop / steps).mean()),
        "epilogue_us": float((t[3] - t[2]).mean()),
        "steps": int(steps.sum()),
    }
    xcds = {}
    for x in sorted(set(xcc.tolist())):
        m = xcc == x
        xcds[int(x)] = {"workgroups": int(m.sum()), "us_per_step": float(loop[m].sum() / steps[m].sum()),
                        "last_end_us": float(t[3][m].max())}
    out["xcd"] = xcds
    by_unit = collections.defaultdict(list)
    for i in range(n):
        by_unit[int(unit[i])].append(i)
    ends = np.array([t[3][v].max() for v in by_unit.values()])
    gaps = []
    for v in by_unit.values():
        # a workgroup that started after others on its unit ended: its start
        # against the latest of those ends (the slot it took)
        for c in v:
            prior = [t[3][i] for i in v if t[3][i] <= t[0][c]]
            if prior:
                gaps.append(t[0][c] - max(prior))
    out["units"] = len(by_unit)
    out["unit_end_us"] = (float(ends.min()), float(np.median(ends)), float(ends.max()))
    out["gap_us"] = float(np.mean(gaps)) if gaps else None
    if n >= 2 * n_cu:
        out["first_wave_us_per_step"] = (float((loop[:n_cu] / steps[:n_cu]).mean()),
                                         float((loop[n_cu:2 * n_cu] / steps[n_cu:2 * n_cu]).mean()))
    return out


def report(name: str, fig: dict, event_us: float) -> str:
    """Markdown lines for one workload's figures."""
    lines = [f"### `{name}`", "",
             f"- {fig['workgroups']} workgroups on {fig['units']} compute units; one launch: "
             f"{fig['span_us']:.1f} us from the first start to the last end "
             f"({event_us:.1f} us by HIP events around it)",
             f"- per workgroup, averages: prologue {fig['prologue_us']:.2f} us, key loop "
             f"{fig['loop_us_per_step']:.3f} us per step, epilogue {fig['epilogue_us']:.2f} us"]
    lo, med, hi = fig["unit_end_us"]
    gap = "" if fig["gap_us"] is None else (
        f"; from a workgroup's end to the next start on its unit: {fig['gap_us']:.2f} us")
    lines.append(f"- compute units end between {lo:.1f} and {hi:.1f} us (median {med:.1f}){gap}")
    if "first_wave_us_per_step" in fig:
        a, c = fig["first_wave_us_per_step"]
        lines.append(f"- first wave, key loop per step: a unit's first workgroup {a:.3f} us, its second "
                     f"{c:.3f} us")
    lines += ["", "| XCD | workgroups | key loop, us per step | last end, us |", "|---|---|---|---|"]
    for x, v in fig["xcd"].items():
        lines.append(f"| {x} | {v['workgroups']} | {v['us_per_step']:.3f} | {v['last_end_us']:.1f} |")
    return "\n".join(lines) + "\n"


def run(names, warmup: int) -> None:
    import torch

    sys.path.insert(0, ROOT)
    import workloads as wl

    if not os.path.exists(TIMELINE_LIB_PATH):
        raise RuntimeError(f"{TIMELINE_LIB_PATH} is not built (timeline build)")
    lib = ctypes.CDLL(TIMELINE_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa2_fwd.restype = i
    lib.fa2_timeline_clear.argtypes = [vp]
    lib.fa2_timeline_read.argtypes = [vp, i]
    cap = lib.fa2_timeline_capacity()
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    by_name = {w.name: w for w in wl.ALL}
    for name in names:
        w = by_name[name]
        q, k, v = (x.to(dev) for x in wl.make_qkv(w, seed=0))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        code = 0 if w.dtype == "f16" else 1

        def call():
            st = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), w.B, w.H, w.S, w.D, int(w.causal), float(w.scale),
                             code, stream)
            assert st == 0, st

        for _ in range(warmup):
            call()
        assert lib.fa2_timeline_clear(stream) == 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        call()
        ev[1].record()
        torch.cuda.synchronize(dev)
        buf = np.zeros(cap * SLOTS, dtype=np.uint64)
        assert lib.fa2_timeline_read(buf.ctypes.data, cap) == 0
        words = buf.reshape(cap, SLOTS)
        n_wg = int(np.count_nonzero(words[:, 3]))
        assert n_wg > 0 and np.count_nonzero(words[n_wg:, 3]) == 0, "stamps missing"
        print(report(name, summarize(words[:n_wg], n_cu), ev[0].elapsed_time(ev[1]) * 1e3),
              flush=True)
        del q, k, v, o, lse


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--workload", action="append", default=None)
    r.add_argument("--warmup", type=int, default=300)
    a = ap.parse_args(argv)
    if a.cmd == "build":
        print(build_timeline(force=True))
    else:
        run(a.workload or ["sweep_s8192_d128", "llm_layer_causal"], a.warmup)


if __name__ == "__main__":
    main()
