"""Seeded synthetic attention workloads.

This module only draws inputs and names shapes. It holds none of the
attention arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from here without sharing any computation.

Inputs follow the pages' benchmark setting: random N(0, 1) Q, K, V in
(batch, heads, seq, head_dim) layout, fp16 or bf16, scale 1/sqrt(head_dim)
(jared-hpc Lecture 6 benchmark task: B=2, H=16, fp16, causal, seqlen
512..16384, head_dim 64/128; cookbook notebook: B=1, H=32, T=2048, D=128).

Recipe: a CPU torch.Generator seeded with `seed` draws q, k, v in that order
as fp32 N(0, 1) tensors of shape (B, H, S, D); when `qk_mult` is not 1, q and
k are multiplied by it in fp32; each tensor is then rounded once to the
working dtype (round to nearest even). The oracle receives exactly those
rounded values, widened to fp64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str  # "f16" or "bf16"
    causal: bool
    qk_mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def flops(self) -> float:
        """4*B*H*S^2*D, halved under causal masking (the benchmark's count)."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once (2 B per element), lse (4 B per row)."""
        n = self.B * self.H * self.S
        return 4 * n * self.D * 2 + n * 4

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def make_qkv(w: Workload, seed: int = 0):
    """Draw (q, k, v) on the CPU in the workload's dtype (see module recipe)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (w.B, w.H, w.S, w.D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


@dataclass(frozen=True)
class DecodeWorkload:
    """Sq queries against Sk cached keys per head (the KV-cache form)."""
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str
    causal: bool
    qk_mult: float = 1.0
    # "e4m3": K and V are FP8 codes with per-tensor descales (else q's dtype)
    kv: str = ""
    k_descale: float = 1.0
    v_descale: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def flops(self) -> float:
        """4 * B * H * Sq * Sk * D over every query-key pair (causal drops
        about Sq^2 / 2 of them, ignored: Sq << Sk)."""
        return 4.0 * self.B * self.H * self.Sq * self.Sk * self.D

    @property
    def algorithmic_bytes(self) -> int:
        """K and V read once (1 byte per element for FP8), Q read once, O
        written once, lse written once."""
        kv = 2 * self.B * self.H * self.Sk * self.D * (1 if self.kv == "e4m3" else 2)
        qo = 2 * self.B * self.H * self.Sq * self.D * 2
        return kv + qo + self.B * self.H * self.Sq * 4


def make_qkv_decode(w: DecodeWorkload, seed: int = 0):
    """q (B, H, Sq, D), then k and v (B, H, Sk, D), drawn in that order as
    fp32 N(0, 1) from one seeded CPU generator, q and k times qk_mult in fp32,
    then rounded once to the dtype (the recipe of make_qkv with two lengths)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((w.B, w.H, w.Sq, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H, w.Sk, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.H, w.Sk, w.D), generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_qkv_decode_fp8(w: DecodeWorkload, seed: int = 0):
    """q as make_qkv_decode draws it, and k and v as FP8 e4m3 codes: the same
    fp32 draws divided by the workload's descales and cast once to
    torch.float8_e4m3fn (round to nearest, saturating at 448). Returns
    (q, k_codes, v_codes); the values they stand for are codes * descale."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((w.B, w.H, w.Sq, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H, w.Sk, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.H, w.Sk, w.D), generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    f8 = torch.float8_e4m3fn
    k8 = (k / w.k_descale).clamp(-448.0, 448.0).to(f8)
    v8 = (v / w.v_descale).clamp(-448.0, 448.0).to(f8)
    return q.to(w.torch_dtype), k8, v8


def fp8_descales(w: Workload):
    """Per-tensor descales of a workload's FP8 inputs: N(0, qk_mult^2) values
    over 1/64 of that spread, so that |x| / descale stays under e4m3's 448
    (about 5.5 standard deviations)."""
    return w.qk_mult / 64.0, w.qk_mult / 64.0, 1.0 / 64.0


def make_qkv_fp8(w: Workload, seed: int = 0):
    """(q, k, v) as FP8 e4m3 codes: the fp32 draws of make_qkv (same
    generator, order and qk_mult), each divided by its descale
    (fp8_descales) and cast once to torch.float8_e4m3fn (round to nearest
    even). The values they stand for are codes * descale."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (w.B, w.H, w.S, w.D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q = q * w.qk_mult
        k = k * w.qk_mult
    dq, dk, dv = fp8_descales(w)
    f8 = torch.float8_e4m3fn
    return tuple((x / d).clamp(-448.0, 448.0).to(f8) for x, d in ((q, dq), (k, dk), (v, dv)))


def dequantize_fp8(codes, descale: float):
    """The values FP8 codes stand for, in fp64 (exact)."""
    return codes.to(torch.float64) * float(descale)


# Decoding against a long KV cache (split-KV path): one new token per
# sequence, and a speculative/chunked step of 16 new tokens, bf16 and fp16.
DECODE = [
    DecodeWorkload("decode_b8_h32_sk32768_d128", 8, 32, 1, 32768, 128, "bf16", True),
    DecodeWorkload("decode_b1_h32_sk131072_d128", 1, 32, 1, 131072, 128, "f16", True),
    DecodeWorkload("decode_b4_h32_sq16_sk16384_d128", 4, 32, 16, 16384, 128, "bf16", True),
]

# The same shapes against an FP8 KV cache (descale 1/64: N(0, 1) values map
# to codes up to about 320 of e4m3's 448).
DECODE_FP8 = [
    DecodeWorkload(w.name + "_kv8", w.B, w.H, w.Sq, w.Sk, w.D, w.dtype, w.causal, kv="e4m3",
                   k_descale=1 / 64, v_descale=1 / 64)
    for w in DECODE
]


# Tiny exact case: B=1, H=2, S=256, D=64, fp16, causal and non-causal.
TINY = [
    Workload("tiny_causal", 1, 2, 256, 64, "f16", True),
    Workload("tiny_noncausal", 1, 2, 256, 64, "f16", False),
]

# Sequence-length x head-dim sweep: B=2, H=16, fp16, causal.
SWEEP = [
    Workload(f"sweep_s{S}_d{D}", 2, 16, S, D, "f16", True)
    for D in (64, 128)
    for S in (512, 1024, 2048, 4096, 8192, 16384)
]

# The headline point of the sweep.
HEADLINE = Workload("sweep_s8192_d128", 2, 16, 8192, 128, "f16", True)

# LLM-layer shape: B=1, H=32, S=2048, D=128, fp16, causal and non-causal.
LLM_LAYER = [
    Workload("llm_layer_causal", 1, 32, 2048, 128, "f16", True),
    Workload("llm_layer_noncausal", 1, 32, 2048, 128, "f16", False),
]

# Long-sequence, low-parallelism prefill: bf16, Q and K scaled x3 (peaky rows).
LONG_PREFILL = Workload("long_prefill", 1, 8, 16384, 128, "bf16", False, qk_mult=3.0)

# Ragged large head dim: S = 4097 is not a tile multiple, D = 256, bf16 causal.
RAGGED_D256 = Workload("ragged_d256", 4, 16, 4097, 256, "bf16", True)

# One GPU's share of the headline when its 32 (b, h) heads are split across 8
# GPUs: 4 heads, 256 workgroups, about one per compute unit, which exposes
# the causal tail imbalance.
ONE_GPU_SHARE = Workload("share_b1_h4_s8192_d128", 1, 4, 8192, 128, "f16", True)

ALL = TINY + SWEEP + LLM_LAYER + [LONG_PREFILL, RAGGED_D256, ONE_GPU_SHARE]

TOLERANCE_O = {"f16": 2e-3, "bf16": 1.6e-2}
TOLERANCE_LSE_REL = 1e-4

# Relative accuracy of the sum inside gfx950's FP8 (e4m3) matrix-core
# product v_mfma_f32_32x32x64_f8f6f4: |result - exact| is at most this times
# (|C_in| + sum of |products|). Not published; measured by
# tests/test_fp8_mfma_gpu.py (worst seen 2^-12.3, on operands spanning the
# whole e4m3 range; 2^-15 on attention-like ones; C_in itself is added
# without loss) and held there with a 2x margin. The FP8 attention path's
# tolerance rests on it.
FP8_MFMA_SUM_REL = 2.0 ** -11


def by_name(name: str) -> Workload:
    for w in ALL:
        if w.name == name:
            return w
    raise KeyError(name)
