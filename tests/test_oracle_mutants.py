"""Plant plausible mistakes in copies of the C oracle and check that the pins
catch every one of them (CPU only; the real oracle is never modified).

Each mutant is the oracle's source with one textual edit, compiled with gcc
into a temporary directory and driven through the same pin checks that the
real oracle passes in test_oracle.py.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# (name, original text, replacement): each a mistake one could make writing
# the definition down.
MUTATIONS = [
    ("scale_dropped", "scores[j] = scale * dot;", "scores[j] = dot;"),
    ("scale_squared", "scores[j] = scale * dot;", "scores[j] = scale * scale * dot;"),
    ("diagonal_masked", "causal ? i + 1 : S", "causal ? (i > 0 ? i : 1) : S"),
    ("mask_reversed", "causal ? i + 1 : S", "causal ? S - i : S"),
    ("no_max_shift_in_exp", "scores[j] = exp(scores[j] - m);", "scores[j] = exp(scores[j]);"),
    ("exp2_for_exp", "scores[j] = exp(scores[j] - m);", "scores[j] = exp2(scores[j] - m);"),
    ("lse_log2", "*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    ("lse_no_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("v_row_of_query", "const double *vj = v + head + j * D;", "const double *vj = v + head + i * D;"),
    ("k_used_as_q", "const double *qi = q + head + i * D;", "const double *qi = k + head + i * D;"),
    ("v_used_as_k", "const double *kj = k + head + j * D;", "const double *kj = v + head + j * D;"),
    ("key_stride_wrong", "const double *kj = k + head + j * D;", "const double *kj = k + head + j;"),
    ("head_offset_transposed", "const long head = (b * H + h) * S * D;",
     "const long head = (h * B + b) * S * D;"),
    ("normalise_by_count", "o_row[d] /= l;", "o_row[d] /= (double)n_keys;"),
    ("normalisation_dropped", "o_row[d] /= l;", "o_row[d] /= 1.0;"),
    ("unweighted_sum", "o_row[d] += e * vj[d];", "o_row[d] += vj[d];"),
    ("first_key_skipped", "for (long j = 0; j < n_keys; ++j) {\n        const double *vj",
     "for (long j = 1; j < n_keys; ++j) {\n        const double *vj"),
]


def _mutant_attn(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    mutated = src.replace(old, new)
    if name == "head_offset_transposed":
        # the row helper needs B for this edit; thread it through its signature
        mutated = mutated.replace("long H, long S, long D, long b, long h, long i,",
                                  "long H, long S, long D, long b, long h, long i, long B,")
        mutated = mutated.replace("oracle_one_row(q, k, v, H, S, D, bh / H, bh % H, i, causal,",
                                  "oracle_one_row(q, k, v, H, S, D, bh / H, bh % H, i, B, causal,")
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    dp = ctypes.POINTER(ctypes.c_double)
    L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
    lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, I, D, I]
    lib.oracle_attention_f64.restype = I

    def attn(q, k, v, causal, scale):
        q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, S, Dh = q.shape
        o = np.empty((B, H, S, Dh))
        lse = np.empty((B, H, S))
        with np.errstate(all="ignore"):
            rc = lib.oracle_attention_f64(*(x.ctypes.data_as(dp) for x in (q, k, v, o, lse)),
                                          B, H, S, Dh, int(causal), float(scale), 1)
        assert rc == 0
        return o, lse

    return attn


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    attn = _mutant_attn(tmp_path, name, old, new)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(attn)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    attn = _mutant_attn(tmp_path, "identity", "scores[j] = scale * dot;", "scores[j] = scale * dot;")
    for check in oracle_pins.ALL_CHECKS:
        check(attn)
