"""The oracle's KV-cache form (Sq queries against Sk keys) against the facts
that pin it, and planted mistakes in copies of it that those facts must catch
(CPU only; the real oracle is never modified)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle_kv_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")


def _attn_kv(q, k, v, causal, scale):
    return oracle.attention_kv_f64(q, k, v, causal, scale)


@pytest.mark.parametrize("check", oracle_kv_pins.ALL_KV_CHECKS, ids=lambda f: f.__name__)
def test_oracle_kv_pin(check):
    check(_attn_kv)


def test_kv_with_equal_lengths_matches_square_entry_point():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 3, 17, 8)) for _ in range(3))
    for causal in (False, True):
        a = oracle.attention_f64(q, k, v, causal, 0.4)
        b = oracle.attention_kv_f64(q, k, v, causal, 0.4)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_kv_error_codes():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(RuntimeError):  # causal with more queries than keys
        oracle.attention_kv_f64(q, q[:, :, :3], q[:, :, :3], True, 1.0)
    with pytest.raises(ValueError):
        oracle.attention_kv_f64(q, q[:, :, :3], q[:, :, :2], False, 1.0)


# (name, original text, replacement): mistakes one could make writing the
# KV-cache form down. Every edit keeps all reads inside the arrays the checks
# pass in (Sq <= Sk where an offset would otherwise run past the end).
KV_MUTATIONS = [
    ("offset_dropped", "causal ? i + (Sk - Sq) + 1 : Sk", "causal ? i + 1 : Sk"),
    ("offset_off_by_one", "causal ? i + (Sk - Sq) + 1 : Sk", "causal ? i + (Sk - Sq) : Sk"),
    ("diagonal_dropped_everywhere", "causal ? i + (Sk - Sq) + 1 : Sk", "causal ? (i + (Sk - Sq) > 0 ? i + (Sk - Sq) : 1) : Sk"),
    ("kv_head_with_query_length", "const long kv_head = (b * H + h) * Sk * D;",
     "const long kv_head = (b * H + h) * Sq * D;"),
    ("query_heads_transposed", "const double *qi = q + ((b * H + h) * Sq + i) * D;",
     "const double *qi = q + (((b + h) % (H > 1 ? H : 1) + b * 0) * Sq + i) * D;"),
    ("first_query_for_all", "const double *qi = q + ((b * H + h) * Sq + i) * D;",
     "const double *qi = q + ((b * H + h) * Sq + 0) * D;"),
    ("scale_dropped", "scores[j] = scale * dot;", "scores[j] = dot;"),
    ("lse_log2", "*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    ("v_row_of_query", "const double *vj = v + kv_head + j * D;", "const double *vj = v + kv_head + (j % Sq) * D;"),
    ("normalise_by_count", "o_row[d] /= l;", "o_row[d] /= (double)n_keys;"),
]


def _mutant_kv(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    dp = ctypes.POINTER(ctypes.c_double)
    L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
    lib.oracle_attention_kv_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, I, D, I]
    lib.oracle_attention_kv_f64.restype = I

    def attn_kv(q, k, v, causal, scale):
        q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, Sq, Dh = q.shape
        Sk = k.shape[2]
        o = np.empty((B, H, Sq, Dh))
        lse = np.empty((B, H, Sq))
        with np.errstate(all="ignore"):
            rc = lib.oracle_attention_kv_f64(*(x.ctypes.data_as(dp) for x in (q, k, v, o, lse)),
                                             B, H, Sq, Sk, Dh, int(causal), float(scale), 1)
        assert rc == 0
        return o, lse

    return attn_kv


@pytest.mark.parametrize("name,old,new", KV_MUTATIONS, ids=[m[0] for m in KV_MUTATIONS])
def test_kv_pins_catch_mutant(tmp_path, name, old, new):
    attn_kv = _mutant_kv(tmp_path, name, old, new)
    caught = []
    for check in oracle_kv_pins.ALL_KV_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(attn_kv)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_kv_unmutated_copy_passes_every_pin(tmp_path):
    attn_kv = _mutant_kv(tmp_path, "identity", "scores[j] = scale * dot;", "scores[j] = scale * dot;")
    for check in oracle_kv_pins.ALL_KV_CHECKS:
        check(attn_kv)
