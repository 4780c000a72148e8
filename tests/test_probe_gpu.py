"""The matrix-core ceiling probe that bench.py reports beside the roofline:
it runs, its clock reading is plausible, and its rate stays under the
nominal dense fp16 peak at that clock."""
import pytest

import bench

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ceiling_probe_rate_and_clock(dtype):
    r = bench.mfma_ceiling(warmup_min_s=0.05, launches=3, dtype=dtype)
    assert r is not None, "libfa2probe.so is not built"
    print(f"[probe] {r}", flush=True)
    assert 0.5 <= r["clock_ghz"] <= 2.6
    # 256 CUs x 4096 FLOP per clock at the measured clock bounds the rate
    assert 0.0 < r["tflops"] <= 256 * 4096 * r["clock_ghz"] * 1e9 / 1e12 * 1.02
    assert r["frac_of_peak"] <= 1.0
