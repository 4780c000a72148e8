"""Seeded random shapes against the fp64 oracle, every output compared.

Hypothesis draws (B, H, S, D, dtype, causal, scale, Q/K magnitude) from
ranges that stay small enough for the oracle to run every case in well under
a second; the draw is derandomized, so a run is reproducible and the failing
case, if any, is printed with its parameters. Inputs come from the same
seeded generator as every other test (workloads.make_qkv). Tolerances are
the parity bar of test_parity_gpu.
"""
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import workloads as wl  # noqa: E402
from gpu_helpers import announce, assert_parity, oracle_full, run_gpu  # noqa: E402

pytestmark = pytest.mark.gpu


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(
    B=st.integers(1, 3),
    H=st.integers(1, 4),
    S=st.integers(1, 320),
    D=st.sampled_from([64, 128, 256]),
    dtype=st.sampled_from(["f16", "bf16"]),
    causal=st.booleans(),
    scale_kind=st.sampled_from(["default", "random"]),
    scale_value=st.floats(0.0, 0.5),
    qk_mult=st.sampled_from([1.0, 2.0, 3.0]),
    seed=st.integers(0, 2**31 - 1),
)
def test_random_shapes(B, H, S, D, dtype, causal, scale_kind, scale_value, qk_mult, seed):
    w = wl.Workload("random", B, H, S, D, dtype, causal, qk_mult=qk_mult)
    scale = w.scale if scale_kind == "default" else scale_value
    what = (f"B={B} H={H} S={S} D={D} {dtype} causal={causal} scale={scale:.4g} "
            f"qk_mult={qk_mult} seed={seed}")
    announce(what)
    q, k, v = wl.make_qkv(w, seed)
    o, lse = run_gpu(q, k, v, causal, scale)
    o_ref, lse_ref = oracle_full(q, k, v, causal, scale)
    assert_parity(o, lse, o_ref, lse_ref, dtype, what)
