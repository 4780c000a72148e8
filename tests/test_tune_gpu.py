"""Every tile-sweep candidate (flashattention_tiled_amd/tune.py) against the
fp64 oracle, not only against the default library: each candidate library
built by `tune build` runs one ragged shape of its head dim (B=1, H=2,
S=1000: several tiles and a partial last one), causal and not, fp16 and
bf16, and every output must meet the parity bar (max |dO| <= 2e-3 fp16 /
1.6e-2 bf16, lse relative error <= 1e-4). Skipped when the candidates have
not been built."""
import os

import pytest
import torch

import flashattention_tiled_amd as fa
from flashattention_tiled_amd import tune
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity, oracle_full

pytestmark = pytest.mark.gpu

OUT = os.path.join(tune.ROOT, "_build", "tune")
BUILT = [(D, cfg) for D, cfgs in tune.CANDIDATES.items() for cfg in cfgs
         if tune.valid(D, cfg) and os.path.exists(os.path.join(OUT, f"libfa2_{tune.name(D, cfg)}.so"))]


@pytest.mark.skipif(not BUILT, reason="tile-sweep candidates not built (tune build)")
@pytest.mark.parametrize("D,cfg", BUILT, ids=lambda x: str(x))
def test_candidate_meets_oracle(D, cfg):
    lib = tune._open(os.path.join(OUT, f"libfa2_{tune.name(D, cfg)}.so"))
    stream = torch.cuda.current_stream().cuda_stream
    for dtype in ("f16", "bf16"):
        for causal in (False, True):
            w = wl.Workload("tune_check", 1, 2, 1000, D, dtype, causal)
            announce(f"candidate {tune.name(D, cfg)} {dtype} causal={causal}")
            q, k, v = wl.make_qkv(w, seed=D)
            qd, kd, vd = (x.to(DEV) for x in (q, k, v))
            o = torch.empty_like(qd)
            lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=DEV)
            st = lib.fa2_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), w.B, w.H, w.S, w.D, int(causal), float(w.scale),
                             fa.FA2_F16 if dtype == "f16" else fa.FA2_BF16, stream)
            assert st == 0
            torch.cuda.synchronize()
            o_ref, lse_ref = oracle_full(q, k, v, causal, w.scale)
            assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype,
                          f"{tune.name(D, cfg)} {dtype} causal={causal}")
