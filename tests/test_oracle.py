"""The fp64 oracle against the facts that pin it (no GPU needed)."""
import numpy as np
import pytest

import oracle
import oracle_pins


def _attn(q, k, v, causal, scale):
    return oracle.attention_f64(q, k, v, causal, scale)


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(_attn)


def test_rows_api_matches_full():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((2, 3, 9, 5)) for _ in range(3))
    rows = np.array([0, 8, 9, 26, 30, 53])  # flat (b*H + h)*S + i
    for causal in (False, True):
        o, lse = oracle.attention_f64(q, k, v, causal, 0.5)
        o_r, lse_r = oracle.attention_rows_f64(q, k, v, rows, causal, 0.5)
        assert np.array_equal(o_r, o.reshape(-1, 5)[rows])
        assert np.array_equal(lse_r, lse.reshape(-1)[rows])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 4, 33, 8)) for _ in range(3))
    a = oracle.attention_f64(q, k, v, True, 0.3, nthreads=1)
    b = oracle.attention_f64(q, k, v, True, 0.3, nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_error_codes():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(TypeError):
        oracle.attention_f64(q.astype(np.float32), q, q, False, 1.0)
    with pytest.raises(ValueError):
        oracle.attention_f64(q, q[:, :, :3], q, False, 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention_rows_f64(q, q, q, [4], False, 1.0)  # row out of range


def test_widening_is_exact():
    """The oracle sees the GPU's fp16/bf16 inputs widened exactly to fp64."""
    import torch
    x = torch.tensor([1.0 / 3.0, 65504.0, 2.0 ** -24, -0.0], dtype=torch.float16)
    assert x.double().tolist() == [0.333251953125, 65504.0, 2.0 ** -24, -0.0]
    y = torch.tensor([1.0 / 3.0], dtype=torch.bfloat16)
    assert y.double().item() == 0.333984375
