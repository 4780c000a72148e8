"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package. The HIP library and its Python binding never do, and the
two share no code: the oracle is the plain definition of attention written in
C (``attn_oracle.c``), one query row at a time, with the full score row held
in memory.

What it follows (the pages' statement of the problem):
  * scores s_ij = scale * q_i . k_j, scale applied before the mask (cookbook
    notebook "FlashAttention-2 in an attention layer", Triton kernel body);
  * causal keeps j <= i (same kernel, causal mask);
  * two-pass softmax, o_i = sum_j exp(s_ij - m_i) v_j / l_i (the standard
    attention that FlashAttention-2 reproduces exactly, infra.bea.ai guide
    introduction);
  * lse_i = m_i + ln l_i (the per-row logsumexp of the FlashAttention-2
    epilogue, jared-hpc Lecture 6 reading task);
  * a KV-cache form with Sq queries against Sk keys, the queries being the
    last Sq positions (causal keeps j <= i + Sk - Sq), for the decoding
    variant the infra.bea.ai guide names ("When V2 Is Used vs Not");
  * beside the definition, the FP8 path's tolerance: a forward error bound
    per output for FP8 products and P rounded to e4m3 (attn_oracle.c).

Inputs are numpy fp64 arrays holding exactly the values the GPU receives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
        lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, I, D, I]
        lib.oracle_attention_f64.restype = I
        lib.oracle_attention_rows_f64.argtypes = [dp, dp, dp, lp, L, dp, dp,
                                                   L, L, L, L, I, D, I]
        lib.oracle_attention_rows_f64.restype = I
        lib.oracle_attention_kv_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, I, D, I]
        lib.oracle_attention_kv_f64.restype = I
        lib.oracle_attention_fp8_bound_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, L, L, L, L,
                                                       I, D, D, D, D, I]
        lib.oracle_attention_fp8_bound_f64.restype = I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        raise TypeError(f"oracle takes fp64 arrays, got {a.dtype}")
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _shape4(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one (B, H, S, D) shape: "
                         f"{q.shape} {k.shape} {v.shape}")
    return q.shape


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attention_f64(q, k, v, causal: bool, scale: float, nthreads: int = 0):
    """Full attention. Returns (o (B,H,S,D), lse (B,H,S)), both fp64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = _shape4(q, k, v)
    o = np.empty((B, H, S, D), np.float64)
    lse = np.empty((B, H, S), np.float64)
    rc = _load().oracle_attention_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      B, H, S, D, int(bool(causal)), float(scale),
                                      int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_f64 failed with code {rc}")
    return o, lse


def attention_rows_f64(q, k, v, rows, causal: bool, scale: float, nthreads: int = 0):
    """Selected rows. `rows` holds flat indices (b*H + h)*S + i.

    Returns (o_rows (n, D), lse_rows (n,)), both fp64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = _shape4(q, k, v)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    n = r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_attention_rows_f64(_ptr(q), _ptr(k), _ptr(v),
                                           _ptr(r, ctypes.c_long), n, _ptr(o), _ptr(lse),
                                           B, H, S, D, int(bool(causal)), float(scale),
                                           int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows_f64 failed with code {rc}")
    return o, lse


def attention_kv_f64(q, k, v, causal: bool, scale: float, nthreads: int = 0):
    """Sq queries against Sk keys per head (the KV-cache form): q (B,H,Sq,D),
    k and v (B,H,Sk,D). Causal keeps key j for query i iff j <= i + Sk - Sq.

    Returns (o (B,H,Sq,D), lse (B,H,Sq)), both fp64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError(f"q (B,H,Sq,D), k and v (B,H,Sk,D): {q.shape} {k.shape} {v.shape}")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    o = np.empty((B, H, Sq, D), np.float64)
    lse = np.empty((B, H, Sq), np.float64)
    rc = _load().oracle_attention_kv_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         B, H, Sq, Sk, D, int(bool(causal)), float(scale),
                                         int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_kv_f64 failed with code {rc}")
    return o, lse


def attention_fp8_bound_f64(q, k, v, causal: bool, scale: float, eps_sum: float, p_exp: float,
                            u_out: float, nthreads: int = 0):
    """Exact attention on the given (dequantized FP8) inputs, and the
    tolerance of the FP8 path per output: a forward error bound for
    products whose sums are within eps_sum of exact (relative to the sum of
    |terms|) and P rounded to e4m3 as 2^(t - m + p_exp), O rounded to an
    output type of relative half-ulp u_out (attn_oracle.c derives it).

    Returns (o, lse, bound_o, bound_lse), fp64, shaped (B,H,S,D) and (B,H,S).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = _shape4(q, k, v)
    o = np.empty((B, H, S, D), np.float64)
    lse = np.empty((B, H, S), np.float64)
    bo = np.empty((B, H, S, D), np.float64)
    bl = np.empty((B, H, S), np.float64)
    rc = _load().oracle_attention_fp8_bound_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                _ptr(bo), _ptr(bl), B, H, S, D,
                                                int(bool(causal)), float(scale), float(eps_sum),
                                                float(p_exp), float(u_out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_fp8_bound_f64 failed with code {rc}")
    return o, lse, bo, bl
