"""Tile sweep for the prefill kernel: the compile-time counterpart of the
cookbook notebook's exercise "Autotune BLOCK_M, BLOCK_N, num_warps".

Each candidate sets one head dim's tile configuration (waves per workgroup,
32-row blocks per wave, keys per tile, waves per SIMD, load spacing and,
optionally, the depth of the K and V LDS rings (2 if absent) and whether the
key loop is pipelined (1 if absent); so B_r = 32 * waves * row blocks and
B_c = keys per tile) through the FA2_TILE_D<D> macro of csrc/fa2_plan.h and
is built into a library of its own (without the library's switches to its
long-sequence D = 64 tile and its key-group D = 128 tile, so that the
candidate itself runs at every shape). On a GPU, every library runs every
benchmark shape of its head dim in fp16 and bf16: first a check that its
output agrees with the default library's (both are within the parity
tolerance of exact attention, so they agree within twice it), then the
timing. The library defaults are the best configurations found this way.

    python -m flashattention_tiled_amd.tune build [--out DIR] [--jobs N]
    python -m flashattention_tiled_amd.tune run [--out DIR] [--csv PATH] [--steps K]
    python -m flashattention_tiled_amd.tune report --csv PATH

`build` needs only hipcc; `run` needs the GPU and the libraries `build`
wrote; `report` prints a markdown summary of a `run` CSV.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import csv
import ctypes
import math
import os
import subprocess
import sys
import time

from .build import CSRC, HIP_FLAGS, HIPCC, INCLUDE, ROOT, SOURCES

# (waves, row blocks, keys per tile, waves per SIMD, load spacing[, stages[,
# pipelined]]); the first entry of each list is the library default
CANDIDATES = {
    64: [(4, 1, 64, 2, 1), (4, 1, 64, 2, 0), (4, 1, 64, 2, 2), (4, 1, 32, 4, 0),
         (4, 1, 32, 2, 0), (8, 1, 64, 2, 0), (2, 1, 64, 2, 0), (4, 2, 64, 1, 0),
         (4, 1, 128, 1, 0)],
    128: [(4, 1, 64, 2, 2), (4, 1, 64, 2, 0), (4, 1, 64, 2, 1), (4, 1, 64, 2, 4),
          (8, 1, 64, 2, 2), (4, 1, 32, 2, 0), (2, 1, 64, 2, 1), (4, 1, 128, 1, 2)],
    256: [(4, 1, 32, 2, 1, 2, 0), (4, 1, 32, 2, 0, 2, 0), (4, 1, 32, 2, 2, 2, 0),
          (8, 1, 32, 2, 1, 2, 0), (8, 1, 32, 2, 1, 4, 0), (4, 1, 64, 1, 1, 2),
          (4, 1, 64, 1, 2, 2), (4, 1, 32, 1, 1, 4), (4, 1, 32, 1, 0, 4)],
}


def valid(D: int, cfg) -> bool:
    """The kernel's compile-time conditions on a configuration."""
    w, rb, bc, wps, le = cfg[:5]
    stages = cfg[5] if len(cfg) > 5 else 2
    if len(cfg) > 6 and cfg[6] not in (0, 1):
        return False
    tile_bytes = bc * D * 2
    if (bc % 32 or tile_bytes % (1024 * w) or 2 * stages * tile_bytes > 160 * 1024
            or w * 64 > 1024 or stages < 2):
        return False
    lpw = tile_bytes // 1024 // w
    if (stages - 2) * 2 * lpw >= 64 or stages > 4:  # the key loop unrolls by at most 6
        return False
    ns1 = (D // 16) * (bc // 32)  # phase-1 k-steps per tile
    return le == 0 or (ns1 + le - 1) // le >= 2 * lpw


def name(D: int, cfg) -> str:
    st = f"_st{cfg[5]}" if len(cfg) > 5 else ""
    serial = "_serial" if len(cfg) > 6 and cfg[6] == 0 else ""
    return f"d{D}_w{cfg[0]}_rb{cfg[1]}_bc{cfg[2]}_wps{cfg[3]}_le{cfg[4]}{st}{serial}"


def _build_one(out: str, D: int, cfg) -> tuple:
    path = os.path.join(out, f"libfa2_{name(D, cfg)}.so")
    val = ",".join(str(x) for x in cfg)
    # the candidate runs at every shape: no switch to the long-sequence D = 64
    # tile, which takes the candidate's configuration too (both D = 64 tiles
    # must have one B_r), nor to D = 128's key-group tile
    macros = [f"-DFA2_TILE_D{D}={val}", "-DFA2_D64_LONG_S=2147483647", "-DFA2_D128_ALT=0"]
    if D == 64:
        macros.append(f"-DFA2_TILE_D64_LONG={val}")
    cmd = [HIPCC, *HIP_FLAGS, *macros, "-I", INCLUDE, "-I", CSRC, "-o", path, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return D, cfg, path if r.returncode == 0 else None, r.stderr[-2000:]


def build(out: str, jobs: int) -> None:
    os.makedirs(out, exist_ok=True)
    todo = [(D, cfg) for D, cfgs in CANDIDATES.items() for cfg in cfgs if valid(D, cfg)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for D, cfg, path, err in ex.map(lambda a: _build_one(out, *a), todo):
            if path:
                print(f"built {name(D, cfg)}", flush=True)
            else:
                print(f"FAILED {name(D, cfg)}: {err.strip().splitlines()[-1] if err else ''}",
                      flush=True)


def _open(path: str):
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)

    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa2_fwd.restype = i
    return lib


def _shapes(D: int):
    """Benchmark shapes of head dim D, plus two D = 256 shapes beside the
    ragged one so that every head dim has a spread of sizes."""
    sys.path.insert(0, ROOT)
    import workloads as wl

    shapes = [w for w in wl.ALL if w.D == D and w.S >= 512]
    if D == 256:
        shapes += [wl.Workload("tune_s8192_d256", 2, 8, 8192, 256, "bf16", True),
                   wl.Workload("tune_s2048_d256", 2, 16, 2048, 256, "f16", True)]
    return shapes


def run(out: str, csv_path: str, steps: int) -> None:
    import torch

    sys.path.insert(0, ROOT)
    import workloads as wl

    dev = torch.device("cuda:0")
    libs = {}
    for D, cfgs in CANDIDATES.items():
        for cfg in cfgs:
            path = os.path.join(out, f"libfa2_{name(D, cfg)}.so")
            if valid(D, cfg) and os.path.exists(path):
                libs[(D, cfg)] = _open(path)
    rows = []
    for D, cfgs in CANDIDATES.items():
        ref_lib = libs.get((D, cfgs[0]))
        if ref_lib is None:
            print(f"d{D}: the default configuration was not built", flush=True)
            continue
        for w0 in _shapes(D):
            for dtype in ("f16", "bf16"):
                w = wl.Workload(w0.name, w0.B, w0.H, w0.S, w0.D, dtype, w0.causal, w0.qk_mult)
                q, k, v = (x.to(dev) for x in wl.make_qkv(w, seed=0))
                code = 0 if dtype == "f16" else 1
                stream = torch.cuda.current_stream(dev).cuda_stream

                def call(lib, o, lse):
                    st = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), w.B, w.H, w.S, w.D, int(w.causal),
                                     float(w.scale), code, stream)
                    if st != 0:
                        raise RuntimeError(f"fa2_fwd status {st}")

                o_ref = torch.empty_like(q)
                lse_ref = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
                call(ref_lib, o_ref, lse_ref)
                for cfg in cfgs:
                    lib = libs.get((D, cfg))
                    if lib is None:
                        continue
                    o = torch.empty_like(q)
                    lse = torch.empty_like(lse_ref)
                    call(lib, o, lse)
                    torch.cuda.synchronize(dev)
                    d_o = (o.float() - o_ref.float()).abs().max().item()
                    d_l = ((lse - lse_ref).abs() / lse_ref.abs().clamp(min=1.0)).max().item()
                    agree = d_o <= 2 * wl.TOLERANCE_O[dtype] and d_l <= 2 * wl.TOLERANCE_LSE_REL
                    t_w = time.perf_counter()
                    while time.perf_counter() - t_w < 0.3:
                        for _ in range(10):
                            call(lib, o, lse)
                        torch.cuda.synchronize(dev)
                    ev = [(torch.cuda.Event(enable_timing=True),
                           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
                    for a, b in ev:
                        a.record()
                        call(lib, o, lse)
                        b.record()
                    torch.cuda.synchronize(dev)
                    durs = sorted(a.elapsed_time(b) for a, b in ev)
                    med = durs[len(durs) // 2]
                    row = dict(D=D, config=name(D, cfg), default=int(cfg == cfgs[0]),
                               workload=w.name, dtype=dtype, causal=int(w.causal),
                               ms=f"{med:.5f}", tflops=f"{w.flops / med / 1e9:.1f}",
                               agrees=int(agree), max_do=f"{d_o:.2e}", lse_rel=f"{d_l:.2e}")
                    rows.append(row)
                    print(",".join(str(x) for x in row.values()), flush=True)
                del q, k, v, o_ref, lse_ref
    with open(csv_path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        wr.writeheader()
        wr.writerows(rows)


def report(csv_path: str) -> str:
    """Per head dim: each configuration's geometric-mean speed relative to the
    default over all shapes and dtypes, and the best configuration per shape."""
    rows = list(csv.DictReader(open(csv_path)))
    out = []
    for D in sorted({int(r["D"]) for r in rows}):
        rs = [r for r in rows if int(r["D"]) == D]
        base = {(r["workload"], r["dtype"]): float(r["ms"]) for r in rs if r["default"] == "1"}
        out.append(f"\n**D = {D}** (time of the default / time of the configuration; "
                   f"geometric mean over {len(base)} shape-dtype pairs)\n")
        out.append("| configuration | geo-mean speed-up | min | max | agrees with default |")
        out.append("|---|---|---|---|---|")
        for cfg in dict.fromkeys(r["config"] for r in rs):
            sp = [base[(r["workload"], r["dtype"])] / float(r["ms"]) for r in rs
                  if r["config"] == cfg and (r["workload"], r["dtype"]) in base]
            ok = all(r["agrees"] == "1" for r in rs if r["config"] == cfg)
            g = math.exp(sum(math.log(x) for x in sp) / len(sp))
            out.append(f"| `{cfg}` | {g:.3f} | {min(sp):.3f} | {max(sp):.3f} | "
                       f"{'yes' if ok else 'NO'} |")
        out.append("")
        out.append("| shape | dtype | default TFLOP/s | best configuration | its TFLOP/s |")
        out.append("|---|---|---|---|---|")
        for key in base:
            cand = [r for r in rs if (r["workload"], r["dtype"]) == key and r["agrees"] == "1"]
            best = min(cand, key=lambda r: float(r["ms"]))
            dflt = next(r for r in cand if r["default"] == "1")
            out.append(f"| {key[0]} | {key[1]} | {dflt['tflops']} | `{best['config']}` | "
                       f"{best['tflops']} |")
    return "\n".join(out)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("what", choices=("build", "run", "report"))
    ap.add_argument("--out", default=os.path.join(ROOT, "_build", "tune"))
    ap.add_argument("--csv", default=os.path.join(ROOT, "_build", "tune", "sweep.csv"))
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--steps", type=int, default=50)
    a = ap.parse_args()
    if a.what == "build":
        build(a.out, a.jobs)
    elif a.what == "run":
        run(a.out, a.csv, a.steps)
    else:
        print(report(a.csv))


if __name__ == "__main__":
    main()
