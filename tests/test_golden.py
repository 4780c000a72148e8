"""The hand-worked attention instance of tests/golden/ against the oracle (CPU)
and against the HIP path (GPU). Its expected values are closed forms of the
definition (tests/golden/make_worked_example.py), independent of both."""
import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "worked_example_s3_d2.json")
sys.path.insert(0, os.path.join(HERE, "golden"))


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def _inputs(g, d_pad):
    """(1, 1, 3, d_pad) fp64 arrays; head dims past the example's 2 are zero,
    which leaves every score and the first two output dims unchanged."""
    out = []
    for name in ("q", "k", "v"):
        a = np.zeros((1, 1, 3, d_pad))
        a[0, 0, :, :2] = np.array(g[name], dtype=np.float64)
        out.append(a)
    return out


def test_fixture_is_what_the_generator_writes():
    import make_worked_example

    assert make_worked_example.build() == _load()


@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_worked_example(causal):
    import oracle

    g = _load()
    exp = g["causal" if causal else "noncausal"]
    q, k, v = _inputs(g, 2)
    o, lse = oracle.attention_f64(q, k, v, causal, g["scale"])
    assert np.abs(o[0, 0] - np.array(exp["o"])).max() <= 1e-13
    assert np.abs(lse[0, 0] - np.array(exp["lse"])).max() <= 1e-13


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gpu_matches_worked_example(causal, dtype):
    import torch

    import flashattention_tiled_amd as fa
    from workloads import TOLERANCE_LSE_REL, TOLERANCE_O

    g = _load()
    exp = g["causal" if causal else "noncausal"]
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    # the example's integer inputs are exact in both dtypes
    q, k, v = (torch.from_numpy(a).to(td).to("cuda:0") for a in _inputs(g, 64))
    o, lse = fa.attention(q, k, v, causal=causal, scale=g["scale"])
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[0, 0]
    lse = lse.cpu().numpy()[0, 0].astype(np.float64)
    print(f"[golden] {dtype} causal={causal}: O={o[:, :2].tolist()} lse={lse.tolist()}", flush=True)
    assert np.abs(o[:, :2] - np.array(exp["o"])).max() <= TOLERANCE_O[dtype]
    assert (o[:, 2:] == 0).all()
    ref = np.array(exp["lse"])
    assert (np.abs(lse - ref) / np.maximum(np.abs(ref), 1.0)).max() <= TOLERANCE_LSE_REL
    if causal:
        # row 0 sees key 0 alone: its output is V[0] exactly
        assert o[0, :2].tolist() == [1.0, 2.0]


# The same instance read as decoding against a KV cache: the last Sq queries
# of the sequence against all three keys, causal with the queries last (query
# i of the Sq sits at position i + 3 - Sq and keeps keys j <= that position).
# Its rows are the causal rows of the square instance.
@pytest.mark.parametrize("sq", [1, 2])
def test_oracle_kv_form_matches_worked_example(sq):
    import oracle

    g = _load()
    exp = g["causal"]
    q, k, v = _inputs(g, 2)
    o, lse = oracle.attention_kv_f64(q[:, :, 3 - sq:], k, v, True, g["scale"])
    assert np.abs(o[0, 0] - np.array(exp["o"][3 - sq:])).max() <= 1e-13
    assert np.abs(lse[0, 0] - np.array(exp["lse"][3 - sq:])).max() <= 1e-13


@pytest.mark.gpu
@pytest.mark.parametrize("sq", [1, 2])
@pytest.mark.parametrize("kv", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("n_split", [1, 3])
def test_gpu_splitkv_matches_worked_example(sq, kv, n_split):
    import torch

    import flashattention_tiled_amd as fa
    from workloads import TOLERANCE_LSE_REL, TOLERANCE_O

    g = _load()
    exp = g["causal"]
    qd = torch.bfloat16 if kv == "bf16" else torch.float16
    q, k, v = (torch.from_numpy(a) for a in _inputs(g, 64))
    q = q[:, :, 3 - sq:].to(qd).to("cuda:0")
    # the integer inputs are exact in fp16, bf16 and e4m3 (descale 1)
    kvd = torch.float8_e4m3fn if kv == "e4m3" else qd
    k, v = k.to(kvd).to("cuda:0"), v.to(kvd).to("cuda:0")
    o, lse = fa.attention_splitkv(q, k, v, causal=True, scale=g["scale"], n_split=n_split)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[0, 0]
    lse = lse.cpu().numpy()[0, 0].astype(np.float64)
    dt = "bf16" if kv == "bf16" else "f16"
    assert np.abs(o[:, :2] - np.array(exp["o"][3 - sq:])).max() <= TOLERANCE_O[dt]
    assert (o[:, 2:] == 0).all()
    ref = np.array(exp["lse"][3 - sq:])
    assert (np.abs(lse - ref) / np.maximum(np.abs(ref), 1.0)).max() <= TOLERANCE_LSE_REL
