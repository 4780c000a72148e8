#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

One step is one fa2_fwd launch over the whole workload (inputs already
resident in HBM). Default workload: B=2, H=16, S=8192, D=128, fp16, causal.
Prints one JSON line on stdout; diagnostics go to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --table PATH [--oracle]   # every benchmark shape: fa2_fwd, and
                                              # fa2_fwd_balanced where it splits; --oracle adds
                                              # the fp64 oracle over every row (time, parity)
    python bench.py --decode-table PATH   # split-KV decode shapes, GB/s
    python bench.py --layer           # attention layer it/s and peak memory
    python bench.py --mfma-ceiling    # matrix-core rate and clock on random fp16 data
    python bench.py --fp8 [--workload NAME]   # the FP8 prefill, against the FP8 peak

Metric: TFLOP/s with FLOPs = 4*B*H*S^2*D, halved for causal masking, and the
fraction of the MI355X dense fp16/bf16 matrix-core peak (256 CUs x 2.4 GHz x
4096 FLOP/clk/CU = 2516.6 TFLOP/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6  # dense fp16 / bf16 MFMA, MI355X
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 MFMA, MI355X (twice the 16-bit rate)
PEAK_HBM_GBS = 8000.0
# Timing protocol of jared-hpc Lecture 6 ("Measure it"): at least 10 warm-up
# launches before the timed ones; the GPU clock also needs some tenths of a
# second of load to settle after idle, hence a time floor on the warm-up.
WARMUP_MIN_LAUNCHES = 10
WARMUP_MIN_S = 0.5
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fa2_fwd_kernel_sweep_s8192_d128_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    from flashattention_tiled_amd.build import prefill_kernel_sha

    return prefill_kernel_sha()


def library_sha() -> str:
    import flashattention_tiled_amd as fa
    try:
        with open(fa.LIB_PATH, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return ""


def read_traffic(workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this workload with the kernel that is built now (the same
    source, or a bit-identical library); else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    # "- key: `value`" lines, possibly followed by a note
    fields = dict(re.findall(r"^- (\w+): `([^`\n]+)`", text, flags=re.M))
    same_source = fields.get("kernel_sources_sha256") == kernel_source_sha()
    same_library = fields.get("library_sha256", "-") == library_sha()
    if not (same_source or same_library):
        return None
    if fields.get("workload") != workload_name:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_gpu(w, steps: int, warmup: int, warmup_min_s: float = 0.0, balanced: bool = False,
             fp8: bool = False):
    """Per-launch HIP-event durations of fa2_fwd on w (balanced: of
    fa2_fwd_balanced, both its kernels when it splits the keys; fp8: of
    fa2_fwd_fp8 on the workload's inputs as e4m3 codes, O in w's dtype)."""
    import torch

    import flashattention_tiled_amd as fa
    import workloads as wl

    dev = torch.device("cuda:0")
    q, k, v = (wl.make_qkv_fp8 if fp8 else wl.make_qkv)(w, seed=0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty((w.B, w.H, w.S, w.D), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dtype = fa.FA2_F16 if w.dtype == "f16" else fa.FA2_BF16
    lib = fa.load_library()
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.S, w.D, int(w.causal), float(w.scale), dtype, stream.cuda_stream)
    entry = lib.fa2_fwd
    if balanced:
        need = fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, int(w.causal))
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        args = args[:9] + (None,) + args[9:12] + (ws.data_ptr(), need, stream.cuda_stream)
        entry = lib.fa2_fwd_balanced
    elif fp8:
        args = args[:11] + tuple(float(d) for d in wl.fp8_descales(w)) + args[11:]
        entry = lib.fa2_fwd_fp8

    def launch():
        st = entry(*args)
        if st != 0:
            raise fa.FA2Error(st, fa.fa2_status_string(st))

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize(dev)
    # the GPU clock ramps up over tens of milliseconds of work: short launches
    # keep warming up until `warmup_min_s` of launches have run
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warmup_min_s:
        for _ in range(20):
            launch()
        torch.cuda.synchronize(dev)

    # per-launch HIP events on the launch stream, plus wall clock over the steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    durs = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))  # ms
    return dict(q=q, k=k, v=v, o=o, lse=lse, wall_s=wall, durs_ms=durs, launch=launch)


def time_gpu_splitkv(w, steps: int, warmup_min_s: float):
    """Per-call HIP-event durations of fa2_fwd_splitkv (both of its kernels)
    on a decode workload, the workspace allocated before the timed region."""
    import torch

    import flashattention_tiled_amd as fa
    import workloads as wl

    dev = torch.device("cuda:0")
    kv8 = w.kv == "e4m3"
    make = wl.make_qkv_decode_fp8 if kv8 else wl.make_qkv_decode
    q, k, v = (x.to(dev) for x in make(w, seed=0))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = fa.load_library()
    n_split = (fa.fa2_splitkv_splits_fp8 if kv8 else fa.fa2_splitkv_splits)(w.B, w.H, w.Sq, w.Sk)
    need = fa.fa2_splitkv_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, n_split)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    dtype = fa.FA2_F16 if w.dtype == "f16" else fa.FA2_BF16
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.Sq, w.Sk, w.D, int(w.causal), float(w.scale))
    tail = (dtype, n_split, ws.data_ptr(), ws.numel(), stream.cuda_stream)
    entry = lib.fa2_fwd_splitkv_fp8 if kv8 else lib.fa2_fwd_splitkv
    args = head + ((float(w.k_descale), float(w.v_descale)) if kv8 else ()) + tail

    def launch():
        st = entry(*args)
        if st != 0:
            raise fa.FA2Error(st, fa.fa2_status_string(st))

    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warmup_min_s:
        for _ in range(20):
            launch()
        torch.cuda.synchronize(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    return n_split, sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


def run_decode_table(path: str, steps: int):
    import workloads as wl

    rows = []
    for w in wl.DECODE + wl.DECODE_FP8:
        n_split, durs = time_gpu_splitkv(w, steps, warmup_min_s=0.3)
        med = durs[len(durs) // 2]
        avg = sum(durs) / len(durs)
        gbs = w.algorithmic_bytes / (med * 1e-3) / 1e9
        line = (f"{w.name},{w.B},{w.H},{w.Sq},{w.Sk},{w.D},{w.dtype},{w.kv or w.dtype},"
                f"{int(w.causal)},{n_split},"
                f"{med * 1e3:.1f},{avg * 1e3:.1f},{durs[0] * 1e3:.1f},{gbs:.1f},"
                f"{100 * gbs / PEAK_HBM_GBS:.2f}")
        log(line)
        rows.append(line)
    with open(path, "w") as f:
        f.write("workload,B,H,Sq,Sk,D,dtype,kv,causal,n_split,us_median,us_avg,us_min,"
                "alg_GBps,pct_hbm_peak\n")
        f.write("\n".join(rows) + "\n")


def run_layer_bench(steps: int):
    """The attention-layer measurements of the cookbook notebook ("FlashAttention-2
    in an attention layer": "Memory growth", "Throughput"): FA2Attention's
    forward passes per second at B=1, T=2048 for its prose shape (32 heads of
    128) and its code shape (16 heads of 64), against a layer that stores the
    T x T scores as SDPA's math backend does (same weights; its products are
    contiguous fp16 matmuls), and the peak allocation of each at T=512 and
    T=2048. Prints one JSON line per shape."""
    import torch
    from torch import nn

    from flashattention_tiled_amd.layer import FA2Attention

    class ScoresAttention(nn.Module):
        """The baseline: scores materialised, fp32 softmax, causal."""

        def __init__(self, ref: FA2Attention):
            super().__init__()
            self.qkv, self.o, self.h, self.d = ref.qkv, ref.o, ref.num_heads, ref.head_dim

        def forward(self, x):
            B, T, _ = x.shape
            qkv = self.qkv(x).view(B, T, 3, self.h, self.d)
            q, k, v = (qkv[:, :, i].transpose(1, 2).contiguous() for i in range(3))
            s = torch.matmul(q, k.transpose(-1, -2).contiguous()).float() / math.sqrt(self.d)
            mask = torch.ones((T, T), dtype=torch.bool, device=x.device).triu_(1)
            p = torch.softmax(s.masked_fill_(mask, float("-inf")), dim=-1).to(x.dtype)
            out = torch.matmul(p, v)
            return self.o(out.transpose(1, 2).reshape(B, T, -1))

    dev = torch.device("cuda:0")

    def its(layer, x):
        with torch.inference_mode():
            for _ in range(5):
                layer(x)
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            for _ in range(steps):
                layer(x)
            torch.cuda.synchronize(dev)
        return steps / (time.perf_counter() - t0)

    def peak_mib(layer, T, d_model):
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        x = torch.randn((1, T, d_model), device=dev, dtype=torch.float16)
        with torch.inference_mode():
            layer(x)
        torch.cuda.synchronize(dev)
        return torch.cuda.max_memory_allocated(dev) / 2 ** 20

    for d_model, heads in ((4096, 32), (1024, 16)):
        torch.manual_seed(0)
        fa2 = FA2Attention(d_model, heads).to(device=dev, dtype=torch.float16)
        ref = ScoresAttention(fa2)
        x = torch.randn((1, 2048, d_model), device=dev, dtype=torch.float16)
        # warm the clock up on the heavier layer first
        t_w = time.perf_counter()
        with torch.inference_mode():
            while time.perf_counter() - t_w < 0.5:
                ref(x)
            torch.cuda.synchronize(dev)
        r_fa2, r_ref = its(fa2, x), its(ref, x)
        mem = {name: {T: peak_mib(m, T, d_model) for T in (512, 2048)}
               for name, m in (("fa2", fa2), ("scores", ref))}
        print(json.dumps({
            "workload": f"layer_b1_t2048_d{d_model}_h{heads}_f16_causal",
            "fa2_it_per_s": round(r_fa2, 1), "scores_it_per_s": round(r_ref, 1),
            "speedup": round(r_fa2 / r_ref, 2),
            "peak_mib": {n: {str(T): round(v, 1) for T, v in m.items()} for n, m in mem.items()},
            "memory_growth_t512_to_t2048": {n: round(m[2048] / m[512], 2) for n, m in mem.items()},
        }), flush=True)
        del fa2, ref, x


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, budget_s: float):
    """Time the fp64 oracle on a random sample of rows of the same workload
    (about `budget_s` of CPU work) and compare those rows with the GPU output."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    rng = np.random.default_rng(0)
    n_rows_total = w.B * w.H * w.S

    def row_flops(rows):
        i = rows % w.S
        keys = (i + 1) if w.causal else np.full_like(i, w.S)
        return float((4.0 * keys * w.D).sum())

    # calibrate on growing samples until one takes >= 0.5 s, then size the
    # timed sample to the budget
    m = 64
    while True:
        probe = rng.integers(0, n_rows_total, size=min(m, n_rows_total))
        t0 = time.perf_counter()
        oracle.attention_rows_f64(qn, kn, vn, probe, w.causal, w.scale, nthreads=cores)
        t = time.perf_counter() - t0
        if t >= 0.5 or m >= n_rows_total:
            break
        m *= 4
    per_flop = t / row_flops(probe)
    mean_row_flops = 4.0 * w.D * ((w.S + 1) / 2 if w.causal else w.S)
    n = int(min(n_rows_total, max(cores, budget_s / (per_flop * mean_row_flops))))
    rows = np.sort(rng.choice(n_rows_total, size=n, replace=False))
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention_rows_f64(qn, kn, vn, rows, w.causal, w.scale,
                                               nthreads=cores)
    dt = time.perf_counter() - t0
    flops = row_flops(rows)
    og = o_gpu.reshape(-1, w.D).cpu()[rows].double().numpy()
    lg = lse_gpu.reshape(-1).cpu()[rows].double().numpy()
    o_err = float(np.abs(og - o_ref).max())
    lse_err = float((np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max())
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=(f"{n} of {n_rows_total} query rows drawn uniformly (seed 0), "
                        f"{flops:.3e} FLOPs in {dt:.1f} s, fp64, {cpu}"),
                seconds=dt, parity_max_abs_o=o_err, parity_lse_rel=lse_err)


def mfma_ceiling(warmup_min_s: float = 0.3, launches: int = 20, dtype: str = "f16"):
    """Rate and clock of the matrix-core ceiling probe (libfa2probe.so): fp16
    (or bf16) 32x32x16 products on random N(0, 1) operands and nothing else,
    two workgroups per compute unit, median of `launches` HIP-event timed
    launches after `warmup_min_s` of warm-up. None when the probe is not
    built."""
    import ctypes

    import torch

    from flashattention_tiled_amd.build import PROBE_LIB_PATH

    if not os.path.exists(PROBE_LIB_PATH):
        return None
    lib = ctypes.CDLL(PROBE_LIB_PATH)  # after torch: shares its HIP runtime
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa2_probe_mfma_ceiling.argtypes = [vp, i, i, vp, vp, i, vp]
    lib.fa2_probe_mfma_ceiling.restype = i
    lib.fa2_probe_mfma_flops.argtypes = [i, i]
    lib.fa2_probe_mfma_flops.restype = ctypes.c_double
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    n_wg, iters = 2 * n_cu, 4096
    g = torch.Generator("cpu").manual_seed(0)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    ops = torch.randn(384 * 8, generator=g).to(tdt).to(dev)
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(n_wg * 4 * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def launch():
        st = lib.fa2_probe_mfma_ceiling(ops.data_ptr(), n_wg, iters, sink.data_ptr(),
                                        clocks.data_ptr(), 0 if dtype == "f16" else 1, stream)
        if st != 0:
            raise RuntimeError(f"fa2_probe_mfma_ceiling status {st}")

    t = time.perf_counter()
    while time.perf_counter() - t < warmup_min_s:
        launch()
        torch.cuda.synchronize(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize(dev)
    med = sorted(a.elapsed_time(b) for a, b in ev)[launches // 2]
    tflops = lib.fa2_probe_mfma_flops(n_wg, iters) / (med * 1e-3) / 1e12
    ck = clocks.view(-1, 2).cpu().double()
    # s_memtime counts shader-clock cycles, s_memrealtime a constant 100 MHz
    ghz = float((ck[:, 0] / ck[:, 1]).mean()) * 0.1
    return {"tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_TFLOPS, 4),
            "clock_ghz": round(ghz, 3), "workgroups": n_wg, "ms": round(med, 4),
            "what": f"{dtype} 32x32x16 matrix-core products on random N(0,1) operands only"}


def gpu_clock_mhz(launch, seconds: float):
    """Median of the GPU clock readings (MHz, amdsmi through
    torch.cuda.clock_rate) taken while `launch` keeps the GPU busy for
    `seconds`; None when the clock cannot be read. amdsmi samples the clock
    over periods of 1/6 s or more, so this is the steady-state clock of the
    same launches, taken right after the timed ones."""
    import torch

    try:
        torch.cuda.clock_rate(0)
    except Exception as e:  # noqa: BLE001
        log(f"[bench] GPU clock not readable: {e}")
        return None
    samples = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            launch()
        samples.append(float(torch.cuda.clock_rate(0)))
        torch.cuda.synchronize()
    samples.sort()
    return samples[len(samples) // 2] if samples else None


def stats_line(w, r):
    durs = r["durs_ms"]
    avg = sum(durs) / len(durs)
    med = durs[len(durs) // 2]
    return avg, med


def oracle_full_leg(w, q, k, v, o_gpu, lse_gpu, threads: int):
    """The fp64 oracle over every row of w on `threads` host threads: wall
    seconds, GFLOP/s under the benchmark's FLOP count, and the parity of the
    GPU output against it over all outputs."""
    import numpy as np

    import oracle

    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention_f64(qn, kn, vn, w.causal, w.scale, nthreads=threads)
    dt = time.perf_counter() - t0
    og = o_gpu.cpu().double().numpy()
    lg = lse_gpu.cpu().double().numpy()
    o_err = float(np.abs(og - o_ref).max())
    lse_err = float((np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max())
    return dict(seconds=dt, threads=threads, gflops=w.flops / dt / 1e9, max_abs_o=o_err,
                lse_rel=lse_err)


def run_table(path: str, steps: int, warmup: int, with_oracle: bool = False):
    """Every benchmark shape through fa2_fwd (and fa2_fwd_balanced where it
    splits the keys, fa2_fwd_fp8 on e4m3 inputs where it has a kernel) into
    a CSV; pct_peak is of the dense peak of the entry's input type (16-bit
    2516.6, FP8 5033.2 TFLOP/s). with_oracle: also the fp64 oracle over every
    row of each 16-bit shape on all host cores (wall time, GFLOP/s, and the
    parity of the fa2_fwd output against it), and the tiny shapes once more
    on one thread."""
    import workloads as wl

    import flashattention_tiled_amd as fa

    cores = len(os.sched_getaffinity(0))
    rows = []
    for w in wl.ALL:
        # fa2_fwd, fa2_fwd_balanced where it splits the keys of this shape,
        # and fa2_fwd_fp8 (e4m3 inputs)
        entries = ["fa2_fwd"]
        if fa.fa2_fwd_balanced_workspace_bytes(w.B, w.H, w.S, w.D, int(w.causal)) > 0:
            entries.append("fa2_fwd_balanced")
        if w not in wl.TINY:
            entries.append("fa2_fwd_fp8")
        for entry in entries:
            fp8 = entry == "fa2_fwd_fp8"
            r = time_gpu(w, steps, warmup, warmup_min_s=0.3, balanced=entry == "fa2_fwd_balanced",
                         fp8=fp8)
            avg, med = stats_line(w, r)
            tf = w.flops / (med * 1e-3) / 1e12
            # FP8 reads 1-byte Q, K, V: its algorithmic bytes and its peak differ
            n = w.B * w.H * w.S
            alg = (3 * n * w.D + 2 * n * w.D + 4 * n) if fp8 else w.algorithmic_bytes
            gbs = alg / (med * 1e-3) / 1e9
            peak = PEAK_FP8_TFLOPS if fp8 else PEAK_TFLOPS
            line = (f"{w.name},{entry},{w.B},{w.H},{w.S},{w.D},{w.dtype},{int(w.causal)},"
                    f"{med:.4f},{avg:.4f},{min(r['durs_ms']):.4f},{tf:.1f},"
                    f"{100 * tf / peak:.2f},{gbs:.1f}")
            if with_oracle and fp8:
                rows.append(line + ",,,,,")
                log(line)
            elif with_oracle:
                legs = [oracle_full_leg(w, r["q"], r["k"], r["v"], r["o"], r["lse"], cores)]
                if w in wl.TINY:
                    legs.append(oracle_full_leg(w, r["q"], r["k"], r["v"], r["o"], r["lse"], 1))
                for g in legs:
                    rows.append(line + f",{g['threads']},{g['seconds']:.3f},{g['gflops']:.2f},"
                                f"{g['max_abs_o']:.3e},{g['lse_rel']:.3e}")
                    log(rows[-1])
            else:
                rows.append(line)
                log(line)
            del r
    with open(path, "w") as f:
        f.write("workload,entry,B,H,S,D,dtype,causal,ms_median,ms_avg,ms_min,tflops,pct_peak,"
                "alg_GBps" + (",oracle_threads,oracle_s,oracle_GFLOPs,max_abs_o,lse_rel"
                              if with_oracle else "") + "\n")
        f.write("\n".join(rows) + "\n")


def run_fp8(w, args):
    """The FP8 prefill (fa2_fwd_fp8) on w's inputs as e4m3 codes (workloads.make_qkv_fp8),
    O in w's dtype: one JSON line with its TFLOP/s under the benchmark's FLOP
    count and its fraction of the dense FP8 peak. A reduced-precision
    variant: never the headline metric, which is the 16-bit path's."""
    r = time_gpu(w, args.steps, max(args.warmup, WARMUP_MIN_LAUNCHES), warmup_min_s=WARMUP_MIN_S,
                 fp8=True)
    avg, med = stats_line(w, r)
    ms_per_step = 1e3 * r["wall_s"] / args.steps
    log(f"[bench] fp8 kernel avg {avg:.4f} ms, median {med:.4f} ms, min {r['durs_ms'][0]:.4f} ms, "
        f"max {r['durs_ms'][-1]:.4f} ms; wall {ms_per_step:.4f} ms/step")
    achieved = w.flops / (avg * 1e-3) / 1e12
    print(json.dumps({
        "metric": "FP8 (e4m3 Q, K, V) attention fwd TFLOP/s and % of FP8 MFMA peak",
        "value": round(w.flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "out_dtype": w.dtype, "flops_per_step": w.flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "kernel_ms_avg": round(avg, 5), "kernel_ms_median": round(med, 5)},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="sweep_s8192_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--table", default=None, help="time every benchmark shape into a CSV")
    ap.add_argument("--oracle", action="store_true",
                    help="with --table: run the fp64 oracle over every row of each shape "
                         "(wall time, GFLOP/s, parity of all outputs)")
    ap.add_argument("--layer", action="store_true",
                    help="time the attention layer against a score-materialising layer")
    ap.add_argument("--decode-table", default=None,
                    help="time the split-KV path on every decode shape into a CSV")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 (e4m3 Q, K, V) prefill on --workload instead: one JSON "
                         "line against the 5.0 PFLOP/s FP8 peak (not the headline metric)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the matrix-core ceiling probe and print its rate and clock")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="leave the matrix-core ceiling probe out of the bench line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (`steps` times), to "
                         "calibrate the HBM byte counters against a known traffic")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the forward pass on one GPU only: the library "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import flashattention_tiled_amd as fa
    import workloads as wl

    fa.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.layer:
        run_layer_bench(args.steps)
        return
    if args.decode_table:
        run_decode_table(args.decode_table, args.steps)
        return
    if args.table:
        run_table(args.table, args.steps, args.warmup, with_oracle=args.oracle)
        return
    if args.mfma_ceiling:
        for dt in ("f16", "bf16"):
            print(json.dumps(mfma_ceiling(dtype=dt)), flush=True)
        return
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x {args.steps} (reads {n} B and writes {n} B per copy)")
        return

    w = wl.by_name(args.workload)
    if args.fp8:
        run_fp8(w, args)
        return
    log(f"[bench] {w} steps={args.steps} warmup={args.warmup}")
    # warm-up: the requested launches, at least WARMUP_MIN_LAUNCHES of them,
    # then more until WARMUP_MIN_S of launches have run, so that the timed
    # launches find the clock settled however short --warmup is
    r = time_gpu(w, args.steps, max(args.warmup, WARMUP_MIN_LAUNCHES), warmup_min_s=WARMUP_MIN_S)
    avg, med = stats_line(w, r)
    clock = gpu_clock_mhz(r.pop("launch"), 0.5)
    ms_per_step = 1e3 * r["wall_s"] / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (avg * 1e-3) / 1e12
    log(f"[bench] kernel avg {avg:.4f} ms, median {med:.4f} ms, min {r['durs_ms'][0]:.4f} ms, "
        f"max {r['durs_ms'][-1]:.4f} ms; wall {ms_per_step:.4f} ms/step; clock {clock} MHz")
    traffic = read_traffic(w.name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, r["q"], r["k"], r["v"], r["o"], r["lse"], args.cpu_budget)
        log(f"[bench] oracle sample: {cpu['sample']}; parity max|dO|={cpu['parity_max_abs_o']:.3e} "
            f"lse_rel={cpu['parity_lse_rel']:.3e}")

    ceiling = None
    if not args.no_ceiling:
        # an auxiliary figure: a failure here must not cost the bench line
        try:
            ceiling = mfma_ceiling(dtype=w.dtype)
        except Exception as e:  # noqa: BLE001
            log(f"[bench] matrix-core ceiling probe failed: {e}")
    if ceiling is not None:
        ceiling["kernel_frac_of_probe"] = round(achieved / ceiling["tflops"], 4)
        log(f"[bench] matrix-core ceiling probe: {ceiling}")

    out = {
        "metric": "attention fwd TFLOP/s and % of fp16 MFMA peak, B=2 H=16 S=8192 D=128 causal",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "qk_mult": w.qk_mult, "scale": w.scale,
                   "flops_per_step": w.flops, "seed": 0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel_ms_avg": round(avg, 5), "kernel_ms_median": round(med, 5),
                     "kernel_ms_min": round(r["durs_ms"][0], 5),
                     "kernel_ms_max": round(r["durs_ms"][-1], 5),
                     "clock_mhz": clock,
                     "warmup_floor": {"launches": WARMUP_MIN_LAUNCHES, "seconds": WARMUP_MIN_S},
                     "mfma_ceiling_probe": ceiling},
        "cpu_baseline": None if cpu is None else {
            k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "parity_sample": None if cpu is None else {
            "max_abs_o": cpu["parity_max_abs_o"], "lse_rel": cpu["parity_lse_rel"],
            "tol_o": wl.TOLERANCE_O[w.dtype], "tol_lse_rel": wl.TOLERANCE_LSE_REL},
        "host": platform.node(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
