"""How exactly gfx950's FP8 matrix-core product sums its terms.

v_mfma_f32_32x32x64_f8f6f4 (both operands OCP e4m3, no block scales)
computes C_in + sum of 64 products per output. Each e4m3 value is an
integer multiple of 2^-9, so every product is an exact multiple of 2^-18 and
the exact result is an int64 sum, compared here with what the instruction
returns. The attention path that runs its products in FP8 takes its
tolerance from the bound measured here:

    |C_out - (C_in + sum_k a_k b_k)| <= FP8_MFMA_SUM_REL * (|C_in| + sum_k |a_k b_k|)

and single products (one nonzero k) must come out exact, which pins the
operand layout and the e4m3 decoding. The operand sets cover attention-like
values, the whole finite e4m3 range (subnormals included), sums that cancel,
one large term among small ones, and a large C_in.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu

NB = 32  # blocks per operand set (32 x 32 outputs of 64 terms each)


def _probe():
    import ctypes

    from flashattention_tiled_amd.build import PROBE_LIB_PATH

    lib = ctypes.CDLL(PROBE_LIB_PATH)  # after torch: shares its HIP runtime
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa2_probe_mfma_fp8.argtypes = [vp, vp, vp, vp, i, vp]
    lib.fa2_probe_mfma_fp8.restype = i
    return lib


def _codes(x):
    """float32 values -> e4m3 codes (uint8) and the exact integers k with
    value = k * 2^-9."""
    f8 = x.clamp(-448, 448).to(torch.float8_e4m3fn)
    vals = f8.to(torch.float64).numpy()
    k = np.rint(vals * 512.0).astype(np.int64)
    assert np.array_equal(k.astype(np.float64) / 512.0, vals)
    return f8.view(torch.uint8), k


def _operand_sets(g):
    def randn(*s):
        return torch.randn(*s, generator=g)

    shape = (NB, 32, 64)
    sets = {}
    sets["normal"] = (randn(*shape) * 4, randn(*shape) * 4, None)
    all_codes = torch.arange(256, dtype=torch.int32)
    finite = all_codes[(all_codes & 0x7F) != 0x7F]
    pick = lambda: finite[torch.randint(0, len(finite), shape, generator=g)].to(torch.uint8) \
        .view(torch.float8_e4m3fn).to(torch.float32)
    sets["whole_range"] = (pick(), pick(), None)
    # pairs of equal and opposite products (k = 2i, 2i + 1) that cancel
    # exactly, and one small pair left over: the exact sum is tiny against
    # the sum of |terms|
    a = randn(*shape) * 8
    b = randn(*shape) * 8
    a[..., 1::2] = a[..., 0::2]
    b[..., 1::2] = -b[..., 0::2]
    a[..., 62:] = randn(NB, 32, 2) * 0.05
    b[..., 62:] = randn(NB, 32, 2) * 0.05
    sets["cancelling"] = (a, b, None)
    a = torch.full(shape, 0.015625) * torch.sign(randn(*shape))
    b = torch.full(shape, 0.015625) * torch.sign(randn(*shape))
    a[..., 7] = 448.0
    b[..., 7] = 256.0
    sets["one_large"] = (a, b, None)
    # one product near the top of the range and the others spread evenly
    # over the 24 binades below it, random mantissas and signs: the small
    # terms sit where an adder narrower than fp32 drops their low bits
    expo = torch.linspace(0, -24, 64).repeat(NB, 32, 1)
    mant = 1 + torch.rand(*shape, generator=g)
    sign = torch.sign(randn(*shape))
    a = sign * mant * torch.exp2(expo / 2 + 8)
    b = (1 + torch.rand(*shape, generator=g)) * torch.exp2(expo / 2 + 8)
    sets["spread_binades"] = (a, b, None)
    c = (torch.randint(-2**20, 2**20, (NB, 32, 32), generator=g).to(torch.float64) * 2.0 ** -8)
    sets["large_c_in"] = (randn(*shape), randn(*shape), c)
    a = torch.zeros(shape)
    b = torch.zeros(shape)
    idx = torch.randint(0, 64, (NB,), generator=g)
    for n in range(NB):
        a[n, :, idx[n]] = pick()[n, :, 0]
        b[n, :, idx[n]] = pick()[n, :, 1]
    sets["single_term"] = (a, b, None)
    return sets


def test_fp8_product_sum_bound():
    lib = _probe()
    g = torch.Generator().manual_seed(2024)
    stream = torch.cuda.current_stream().cuda_stream
    worst = {}
    for name, (a, b, c) in _operand_sets(g).items():
        announce(f"fp8 product probe: {name}")
        ca, ka = _codes(a)
        cb, kb = _codes(b)
        if c is None:
            c = torch.zeros((NB, 32, 32), dtype=torch.float64)
        c32 = c.to(torch.float32)
        assert torch.equal(c32.double(), c)  # C_in exact in fp32
        kc = np.rint(c.numpy() * 2.0 ** 18).astype(np.int64)
        assert np.array_equal(kc.astype(np.float64) * 2.0 ** -18, c.numpy())
        # exact results and the sum of |terms|, as integers times 2^-18
        prod = np.einsum("nik,njk->nijk", ka, kb)
        exact = (prod.sum(-1) + kc).astype(np.float64) * 2.0 ** -18
        mag = (np.abs(prod).sum(-1) + np.abs(kc)).astype(np.float64) * 2.0 ** -18
        out = torch.empty((NB, 32, 32), dtype=torch.float32, device=DEV)
        da, db, dc = (x.contiguous().to(DEV) for x in (ca, cb, c32))
        st = lib.fa2_probe_mfma_fp8(da.data_ptr(), db.data_ptr(), dc.data_ptr(), out.data_ptr(),
                                    NB, stream)
        assert st == 0
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        err = np.abs(got - exact)
        ratio = np.where(mag > 0, err / np.where(mag > 0, mag, 1.0), err)
        worst[name] = float(ratio.max())
        terms = (np.abs(prod).sum(-1)).astype(np.float64) * 2.0 ** -18
        r_terms = float(np.where(terms > 0, err / np.where(terms > 0, terms, 1.0), err).max())
        r_out = float((err / np.maximum(np.abs(got), 2.0 ** -126)).max())
        print(f"[fp8 sum] {name}: max |err| / (|C_in| + sum|terms|) = {worst[name]:.3e} "
              f"(2^{np.log2(max(worst[name], 1e-300)):.2f}); / sum|terms| = {r_terms:.3e}; "
              f"/ |C_out| = {r_out:.3e}; bound {wl.FP8_MFMA_SUM_REL:.3e}", flush=True)
    assert worst["single_term"] == 0.0, "single e4m3 products must be exact"
    for name, r in worst.items():
        assert r <= wl.FP8_MFMA_SUM_REL, (name, r)


def test_fp8_conversion_rounds_to_nearest_even():
    """v_cvt_pk_fp8_f32, which rounds P in the FP8 attention kernel, gives
    torch.float8_e4m3fn's codes (OCP e4m3, round to nearest even) bit for
    bit on the values P takes: every e4m3 value, the midpoints between
    neighbours (ties), points a quarter and three quarters of the way, and
    random values over [2^-12, 448] (subnormals included)."""
    import ctypes

    from flashattention_tiled_amd.build import PROBE_LIB_PATH

    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa2_probe_cvt_fp8.argtypes = [vp, vp, i, vp]
    lib.fa2_probe_cvt_fp8.restype = i
    announce("fp8 conversion probe")
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    vals = vals[vals <= 448]
    mids = [(vals[:-1] + vals[1:]) * f for f in (0.5,)]
    quarters = [vals[:-1] * (1 - f) + vals[1:] * f for f in (0.25, 0.75)]
    g = torch.Generator().manual_seed(7)
    rand = torch.exp2(torch.rand(4096, generator=g, dtype=torch.float64) * 20.8 - 12.0)
    x = torch.cat([vals, *mids, *quarters, rand.clamp(max=448.0)]).to(torch.float32)
    x = torch.cat([x, torch.zeros((-len(x)) % 4)])
    xd = x.to(DEV)
    out = torch.empty(len(x), dtype=torch.uint8, device=DEV)
    assert lib.fa2_probe_cvt_fp8(xd.data_ptr(), out.data_ptr(), len(x),
                                 torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = x.to(torch.float8_e4m3fn).view(torch.uint8)
    bad = (out.cpu() != want).nonzero().flatten()
    assert len(bad) == 0, [(float(x[j]), int(out[j]), int(want[j])) for j in bad[:8]]
