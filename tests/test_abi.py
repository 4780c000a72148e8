"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before touching a device.

Pointers here are plain integers that are never dereferenced: every case
below returns during argument validation, before any HIP call.
"""
import ctypes
import os
import re

import pytest

import flashattention_tiled_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa2_\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from flashattention_tiled_amd.build import build_library
        build_library(force=False)
    return fa.load_library()


def test_header_declares_expected_functions():
    assert sorted(_declared_functions()) == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"libfa2.so does not export {name}"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _elf_dynamic(path):
    """(NEEDED libraries, defined global function names) of a shared object,
    read with binutils."""
    import subprocess

    dyn = subprocess.run(["readelf", "-d", path], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", dyn)
    syms = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                          check=True).stdout
    defined = [ln.split()[-1] for ln in syms.splitlines() if re.match(r"^\S+ T ", ln)]
    return needed, defined


def test_library_exports_only_the_declared_functions(lib):
    _, defined = _elf_dynamic(fa.LIB_PATH)
    ours = sorted(n for n in defined if n.startswith("fa2"))
    assert ours == sorted(_declared_functions())
    # internal helpers stay hidden
    assert not [n for n in defined if "check_device" in n or "overlaps" in n]


def test_product_path_is_independent_of_the_oracle(lib):
    # the HIP library links no oracle code and its sources include none
    needed, defined = _elf_dynamic(fa.LIB_PATH)
    assert not [n for n in needed if "oracle" in n]
    assert not [n for n in defined if "oracle" in n]
    csrc = os.path.join(ROOT, "flashattention_tiled_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert "oracle" not in text, name
    # the Python binding neither imports nor names the oracle package
    pkg = os.path.join(ROOT, "flashattention_tiled_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            text = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), name


def test_library_shares_torchs_hip_runtime():
    """Loading the library first thing in a process (as a test module's
    collection can) still maps one HIP runtime, torch's: the device pointers
    and streams the library is given come from torch's."""
    import subprocess
    import sys

    code = ("import flashattention_tiled_amd as fa; fa.load_library(); "
            "print('\\n'.join(fa._hip_runtimes_mapped()))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                         text=True, check=True).stdout.split()
    assert len(out) == 1 and "torch" in out[0], out


def test_enums_match_header():
    text = open(HEADER).read()
    for name, value in re.findall(r"(FA2_\w+)\s*=\s*(\d+)", text):
        assert getattr(fa, name) == int(value), name


def test_supported_and_rows(lib):
    for D in (64, 128, 256):
        for dt in (fa.FA2_F16, fa.FA2_BF16):
            assert fa.fa2_supported(D, dt) == 1
        assert fa.fa2_rows_per_workgroup(D) > 0
    for D in (0, 32, 96, 512):
        assert fa.fa2_supported(D, fa.FA2_F16) == 0
        assert fa.fa2_rows_per_workgroup(D) == 0
    assert fa.fa2_supported(128, 2) == 0


def test_status_strings(lib):
    for s in range(12):
        assert fa.fa2_status_string(s)
    assert fa.fa2_status_string(0) == "ok"
    assert "unknown" in fa.fa2_status_string(99)


# Fake, 256-byte aligned, non-overlapping addresses for a (1, 1, 64, 64) problem.
_N = 64 * 64 * 2
Q, K, V, O, L = (0x10000000 + i * 0x100000 for i in range(5))


def _call(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, S=64, D=64, causal=0, scale=0.125,
                dtype=fa.FA2_F16, stream=None)
    args.update(kw)
    return fa.fa2_fwd(**args)


_FWD_CASES = [
    (dict(q=None), fa.FA2_ERR_NULL),
    (dict(k=0), fa.FA2_ERR_NULL),
    (dict(v=None), fa.FA2_ERR_NULL),
    (dict(o=None), fa.FA2_ERR_NULL),
    (dict(lse=None), fa.FA2_ERR_NULL),
    (dict(B=0), fa.FA2_ERR_SHAPE),
    (dict(H=0), fa.FA2_ERR_SHAPE),
    (dict(S=0), fa.FA2_ERR_SHAPE),
    (dict(S=-5), fa.FA2_ERR_SHAPE),
    (dict(B=65536), fa.FA2_ERR_SHAPE),
    (dict(H=70000), fa.FA2_ERR_SHAPE),
    (dict(B=65535, H=65535, S=2**31 - 1, D=256), fa.FA2_ERR_SHAPE),
    (dict(D=32), fa.FA2_ERR_HEADDIM),
    (dict(D=96), fa.FA2_ERR_HEADDIM),
    (dict(D=512), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE),
    (dict(dtype=-1), fa.FA2_ERR_DTYPE),
    (dict(q=Q + 8), fa.FA2_ERR_ALIGN),
    (dict(o=O + 2), fa.FA2_ERR_ALIGN),
    (dict(lse=L + 2), fa.FA2_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA2_ERR_SCALE),
    (dict(scale=float("inf")), fa.FA2_ERR_SCALE),
    (dict(o=Q), fa.FA2_ERR_ALIAS),
    (dict(o=K + 16), fa.FA2_ERR_ALIAS),
    (dict(lse=V + _N - 4), fa.FA2_ERR_ALIAS),
    (dict(lse=O + 64), fa.FA2_ERR_ALIAS),
]


@pytest.mark.parametrize("kw,status", _FWD_CASES)
def test_validation_status(lib, kw, status):
    assert _call(**kw) == status


def test_validation_happens_before_device_lookup(lib):
    # Errors in several arguments report the first check in documented order
    # and never reach the device: no GPU is needed to get them.
    assert _call(q=None, D=3) == fa.FA2_ERR_NULL
    assert _call(S=0, D=3) == fa.FA2_ERR_SHAPE


def test_attention_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention(x, x, x)
    with pytest.raises(ValueError):
        fa.attention(x, x, x[:, :, :4])


def test_no_device_status_without_gpu(lib):
    """On a host with no GPU a fully valid call reports FA2_ERR_NO_DEVICE.
    (Skipped where a GPU exists: these fake addresses must never reach a kernel.)"""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call() == fa.FA2_ERR_NO_DEVICE


def test_heads_past_2gib_are_valid(lib):
    """A head of K and V may span more than 2 GiB (tiles are addressed from
    64-bit starts): S = 2000 rows 2^20 elements apart (4 GiB) get as far as
    the device lookup, and so does a decode against 2^23 + 5 keys; an
    element count past int64 is refused."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    S, D = 2000, 64
    far = [x << 40 for x in range(1, 6)]  # q, k, v, o, lse far apart
    st = [S * D, S * D, D, S << 20, S << 20, 1 << 20, S << 20, S << 20, 1 << 20,
          S * D, S * D, D]
    assert fa.fa2_fwd_strided(far[0], far[1], far[2], far[3], far[4], 1, 1, S, D, st, 1, 0.125,
                              fa.FA2_F16, None) == fa.FA2_ERR_NO_DEVICE
    ws = fa.fa2_splitkv_workspace_bytes(1, 1, 3, (1 << 23) + 5, 128, 4)
    assert fa.fa2_fwd_splitkv(far[0], far[1], far[2], far[3], far[4], 1, 1, 3, (1 << 23) + 5,
                              128, 1, 0.125, fa.FA2_F16, 4, 6 << 40, ws,
                              None) == fa.FA2_ERR_NO_DEVICE
    assert fa.fa2_fwd(far[0], far[1], far[2], far[3], far[4], 65535, 65535, 2**31 - 1, 256, 0,
                      0.125, fa.FA2_F16, None) == fa.FA2_ERR_SHAPE


@pytest.mark.parametrize("scale", [-0.125, -1.0 / 64 ** 0.5, -0.0, -1e30])
def test_negative_scale_is_valid(lib, scale):
    """Any finite scale passes validation, negative ones included: the
    prefill, key-split and split-KV calls all get as far as the device
    lookup (no GPU here: FA2_ERR_NO_DEVICE)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call(scale=scale) == fa.FA2_ERR_NO_DEVICE
    assert _call_strided(scale=scale) == fa.FA2_ERR_NO_DEVICE
    assert _call_balanced(True, scale=scale) == fa.FA2_ERR_NO_DEVICE
    assert _call_splitkv(scale=scale) == fa.FA2_ERR_NO_DEVICE
    assert _call_splitkv_fp8(scale=scale) == fa.FA2_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# strided entry point: B=2, H=3, S=100, D=64
# ---------------------------------------------------------------------------
_B, _H, _S = 2, 3, 100
_CONTIG = [_H * _S * 64, _S * 64, 64] * 4
_BSHD = [_S * _H * 64, 64, _H * 64] * 4
SQ, SK, SV, SO, SL = (0x40000000 + i * 0x1000000 for i in range(5))


def _call_strided(**kw):
    args = dict(q=SQ, k=SK, v=SV, o=SO, lse=SL, B=_B, H=_H, S=_S, D=64, strides=list(_CONTIG),
                causal=0, scale=0.125, dtype=fa.FA2_F16, stream=None)
    args.update(kw)
    return fa.fa2_fwd_strided(**args)


def _with(base, **idx):
    out = list(base)
    for name, val in idx.items():
        out[int(name[1:])] = val
    return out


_STRIDED_CASES = [
    (dict(q=None), fa.FA2_ERR_NULL),
    (dict(strides=None), fa.FA2_ERR_NULL),
    (dict(S=0), fa.FA2_ERR_SHAPE),
    (dict(D=96), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE),
    (dict(strides=_with(_CONTIG, s0=-8)), fa.FA2_ERR_STRIDE),          # negative
    (dict(strides=_with(_CONTIG, s4=4)), fa.FA2_ERR_STRIDE),           # not 16-byte rows
    (dict(strides=_with(_CONTIG, s5=32)), fa.FA2_ERR_STRIDE),          # k rows overlap (< D)
    (dict(strides=_with(_CONTIG, s1=(1 << 40) + 8)), fa.FA2_ERR_STRIDE),
    (dict(strides=_with(_CONTIG, s10=64)), fa.FA2_ERR_STRIDE),         # o heads share rows
    (dict(strides=_with(_CONTIG, s9=0)), fa.FA2_ERR_STRIDE),           # o batch broadcast
    (dict(strides=_with(_CONTIG, s11=64 + 8, s10=100 * 64)), fa.FA2_ERR_STRIDE),  # rows spill into next head
    (dict(strides=_with(_CONTIG, s5=1 << 23)), fa.FA2_ERR_SHAPE),      # 256 K rows span 2^32 B
    (dict(strides=_with(_CONTIG, s2=1 << 23)), fa.FA2_ERR_SHAPE),      # 256 Q rows span 2^32 B
    (dict(strides=_with(_CONTIG, s8=1 << 22)), fa.FA2_ERR_SHAPE),      # 256 V rows span 2^31 B
    (dict(k=SK + 8), fa.FA2_ERR_ALIGN),
    (dict(lse=SL + 2), fa.FA2_ERR_ALIGN),
    (dict(scale=float("inf")), fa.FA2_ERR_SCALE),
    (dict(o=SQ + 1024), fa.FA2_ERR_ALIAS),
    (dict(lse=SV + 4096), fa.FA2_ERR_ALIAS),
]


@pytest.mark.parametrize("kw,status", _STRIDED_CASES)
def test_strided_validation_status(lib, kw, status):
    assert _call_strided(**kw) == status


@pytest.mark.parametrize("strides", [
    _CONTIG, _BSHD,
    _with(_CONTIG, s3=0, s4=0, s6=0, s7=0),          # one K/V shared by every (b, h)
    _with(_BSHD, s9=_S * (_H * 64 + 64), s11=_H * 64 + 64),  # padded o rows
], ids=["contiguous", "bshd", "kv_broadcast", "padded_o"])
def test_strided_valid_layouts_reach_the_device_check(lib, strides):
    """Valid layouts pass every check before the device lookup (no GPU here:
    FA2_ERR_NO_DEVICE; skipped where a GPU exists, the pointers are fake)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call_strided(strides=strides) == fa.FA2_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# balanced (key-split) entry point: fa2_fwd's checks with strides NULL,
# fa2_fwd_strided's with strides, in the same order; the workspace is
# checked after the device (the split depends on its compute units)
# ---------------------------------------------------------------------------
def _call_balanced(strided, **kw):
    if strided:
        args = dict(q=SQ, k=SK, v=SV, o=SO, lse=SL, B=_B, H=_H, S=_S, D=64,
                    strides=list(_CONTIG))
    else:
        args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, S=64, D=64, strides=None)
    args.update(causal=0, scale=0.125, dtype=fa.FA2_F16, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(kw)
    return fa.fa2_fwd_balanced(**args)


@pytest.mark.parametrize("kw,status", _FWD_CASES)
def test_balanced_validation_status(lib, kw, status):
    assert _call_balanced(False, **kw) == status


@pytest.mark.parametrize("kw,status", [c for c in _STRIDED_CASES if "strides" not in c[0]
                                       or c[0]["strides"] is not None])
def test_balanced_strided_validation_status(lib, kw, status):
    assert _call_balanced(True, **kw) == status


def test_balanced_valid_calls_reach_the_device_check(lib):
    """Valid calls, with or without strides and with no workspace, pass every
    check before the device lookup (no GPU here: FA2_ERR_NO_DEVICE)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call_balanced(False) == fa.FA2_ERR_NO_DEVICE
    assert _call_balanced(True) == fa.FA2_ERR_NO_DEVICE
    assert _call_balanced(True, strides=list(_BSHD), causal=1) == fa.FA2_ERR_NO_DEVICE


def test_balanced_workspace_bytes_without_a_device(lib):
    """The split depends on the device's compute units: with no device, or
    with arguments out of range, the size is 0."""
    import torch
    assert fa.fa2_fwd_balanced_workspace_bytes(1, 4, 8192, 96, 1) == 0
    assert fa.fa2_fwd_balanced_workspace_bytes(0, 4, 8192, 128, 1) == 0
    assert fa.fa2_fwd_balanced_workspace_bytes(1, 4, -1, 128, 1) == 0
    if torch.cuda.device_count() == 0:
        assert fa.fa2_fwd_balanced_workspace_bytes(1, 4, 8192, 128, 1) == 0


# ---------------------------------------------------------------------------
# split-KV entry point: (1, 1, Sq=4, 64) queries against Sk=256 keys, D=64
# ---------------------------------------------------------------------------
_SQ, _SK, _D = 4, 256, 64
_NQ, _NKV = _SQ * _D * 2, _SK * _D * 2
QS, KS, VS, OS, LS, WS = (0x20000000 + i * 0x100000 for i in range(6))


def _ws_bytes(n_split):
    return fa.fa2_splitkv_workspace_bytes(1, 1, _SQ, _SK, _D, n_split)


def _call_splitkv(**kw):
    args = dict(q=QS, k=KS, v=VS, o=OS, lse=LS, B=1, H=1, Sq=_SQ, Sk=_SK, D=_D, causal=0,
                scale=0.125, dtype=fa.FA2_F16, n_split=4, workspace=WS,
                workspace_bytes=_ws_bytes(4), stream=None)
    args.update(kw)
    return fa.fa2_fwd_splitkv(**args)


def test_splitkv_workspace_bytes(lib):
    # part_o (B*H*n_split*Sq*D floats, rounded up to 256 bytes) + (m, l, l) per row and chunk
    for B, H, Sq, Sk, D, n in ((1, 1, 1, 100, 64, 1), (2, 3, 5, 999, 128, 7), (1, 2, 33, 64, 256, 3)):
        o_bytes = B * H * n * Sq * D * 4
        expect = (o_bytes + 255) // 256 * 256 + B * H * n * Sq * 3 * 4
        assert fa.fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n) == expect
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 1, 1, 96, 1) == 0
    assert fa.fa2_splitkv_workspace_bytes(0, 1, 1, 1, 64, 1) == 0
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 1, 1, 64, -1) == 0
    assert fa.fa2_splitkv_splits(1, 1, 1, 1 << 20) >= 1
    assert fa.fa2_splitkv_splits(0, 1, 1, 1) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA2_ERR_NULL),
    (dict(lse=None), fa.FA2_ERR_NULL),
    (dict(Sq=0), fa.FA2_ERR_SHAPE),
    (dict(Sk=0), fa.FA2_ERR_SHAPE),
    (dict(B=65536), fa.FA2_ERR_SHAPE),
    (dict(n_split=-1), fa.FA2_ERR_SHAPE),
    (dict(n_split=70000, workspace_bytes=1 << 40), fa.FA2_ERR_SHAPE),
    (dict(causal=1, Sq=_SK + 1), fa.FA2_ERR_SHAPE),
    (dict(B=65535, H=65535, Sk=2**31 - 1), fa.FA2_ERR_SHAPE),  # elements past int64
    (dict(D=96), fa.FA2_ERR_HEADDIM),
    (dict(dtype=3), fa.FA2_ERR_DTYPE),
    (dict(k=KS + 8), fa.FA2_ERR_ALIGN),
    (dict(lse=LS + 1), fa.FA2_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA2_ERR_SCALE),
    (dict(workspace=None), fa.FA2_ERR_WORKSPACE),
    (dict(workspace=WS + 4), fa.FA2_ERR_WORKSPACE),
    (dict(workspace_bytes=_ws_bytes(4) - 1), fa.FA2_ERR_WORKSPACE),
    (dict(n_split=8), fa.FA2_ERR_WORKSPACE),  # the workspace is sized for 4 chunks
    (dict(o=QS), fa.FA2_ERR_ALIAS),
    (dict(lse=KS + _NKV - 4), fa.FA2_ERR_ALIAS),
    (dict(workspace=VS + 16), fa.FA2_ERR_ALIAS),
    (dict(workspace=OS), fa.FA2_ERR_ALIAS),
])
def test_splitkv_validation_status(lib, kw, status):
    assert _call_splitkv(**kw) == status


def _call_splitkv_noalloc(**kw):
    args = dict(q=QS, k=KS, v=VS, o=OS, lse=LS, B=1, H=1, Sq=_SQ, Sk=_SK, D=_D, causal=0,
                scale=0.125, dtype=fa.FA2_F16, n_split=4, stream=None)
    args.update(kw)
    return fa.fa2_fwd_splitkv_noalloc(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA2_ERR_NULL),
    (dict(Sq=0), fa.FA2_ERR_SHAPE),
    (dict(causal=1, Sq=_SK + 1), fa.FA2_ERR_SHAPE),
    (dict(n_split=-1), fa.FA2_ERR_SHAPE),
    (dict(D=96), fa.FA2_ERR_HEADDIM),
    (dict(dtype=2), fa.FA2_ERR_DTYPE),
    (dict(k=KS + 8), fa.FA2_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA2_ERR_SCALE),
    # 64 x 64 heads x 8 chunks x 64 rows x (256 + 3) floats: far past the scratch
    (dict(B=64, H=64, Sq=64, Sk=4096, D=256, n_split=8), fa.FA2_ERR_SCRATCH),
    # just past it: 1 x 1 x n chunks x 4 rows x 67 floats > 16 MiB
    (dict(n_split=(16 << 20) // (4 * 67 * 4) + 1), fa.FA2_ERR_SCRATCH),
])
def test_splitkv_noalloc_validation(lib, kw, status):
    """The no-allocation split-KV call checks its arguments as fa2_fwd_splitkv
    does, and refuses a call whose partials need more than the fixed scratch
    before it looks at the device."""
    assert _call_splitkv_noalloc(**kw) == status


def test_splitkv_noalloc_reaches_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call_splitkv_noalloc() == fa.FA2_ERR_NO_DEVICE
    assert _call_splitkv_noalloc(n_split=0) == fa.FA2_ERR_NO_DEVICE
    assert "scratch" in fa.fa2_status_string(fa.FA2_ERR_SCRATCH)


def _call_splitkv_fp8(**kw):
    args = dict(q=QS, k=KS, v=VS, o=OS, lse=LS, B=1, H=1, Sq=_SQ, Sk=_SK, D=_D, causal=0,
                scale=0.125, k_descale=0.01, v_descale=0.02, dtype=fa.FA2_F16, n_split=4,
                workspace=WS, workspace_bytes=_ws_bytes(4), stream=None)
    args.update(kw)
    return fa.fa2_fwd_splitkv_fp8(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), fa.FA2_ERR_NULL),
    (dict(Sk=0), fa.FA2_ERR_SHAPE),
    (dict(causal=1, Sq=_SK + 1), fa.FA2_ERR_SHAPE),
    (dict(dtype=5), fa.FA2_ERR_DTYPE),
    (dict(D=32), fa.FA2_ERR_HEADDIM),
    (dict(v=VS + 4), fa.FA2_ERR_ALIGN),
    (dict(k_descale=0.0), fa.FA2_ERR_SCALE),
    (dict(v_descale=-1.0), fa.FA2_ERR_SCALE),
    (dict(k_descale=float("nan")), fa.FA2_ERR_SCALE),
    (dict(v_descale=float("inf")), fa.FA2_ERR_SCALE),
    (dict(workspace_bytes=_ws_bytes(4) - 1), fa.FA2_ERR_WORKSPACE),
    (dict(o=KS + 8 * _D), fa.FA2_ERR_ALIAS),
])
def test_splitkv_fp8_validation_status(lib, kw, status):
    assert _call_splitkv_fp8(**kw) == status


def test_splitkv_fp8_kv_extent_is_one_byte_per_element(lib):
    # o just past the FP8 K (Sk * D bytes) does not overlap it; one element
    # earlier does
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call_splitkv_fp8(o=KS + _SK * _D) == fa.FA2_ERR_NO_DEVICE
    assert _call_splitkv_fp8(o=KS + _SK * _D - 16) == fa.FA2_ERR_ALIAS


_SKV_CONTIG = [_SQ * _D, _SQ * _D, _D, _SK * _D, _SK * _D, _D, _SK * _D, _SK * _D, _D,
               _SQ * _D, _SQ * _D, _D]


def _call_splitkv_strided(**kw):
    args = dict(q=QS, k=KS, v=VS, o=OS, lse=LS, B=1, H=1, Sq=_SQ, Sk=_SK, D=_D,
                strides=list(_SKV_CONTIG), causal=0, scale=0.125, dtype=fa.FA2_F16, kv_fp8=0,
                k_descale=1.0, v_descale=1.0, n_split=4, workspace=WS,
                workspace_bytes=_ws_bytes(4), stream=None)
    args.update(kw)
    return fa.fa2_fwd_splitkv_strided(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(strides=None), fa.FA2_ERR_NULL),
    (dict(q=None), fa.FA2_ERR_NULL),
    (dict(kv_fp8=2), fa.FA2_ERR_DTYPE),
    (dict(strides=_with(_SKV_CONTIG, s5=32)), fa.FA2_ERR_STRIDE),       # k rows overlap (< D)
    (dict(strides=_with(_SKV_CONTIG, s0=4)), fa.FA2_ERR_STRIDE),        # q rows not 16-byte aligned
    (dict(strides=_with(_SKV_CONTIG, s5=72), kv_fp8=1, k_descale=0.1,
          v_descale=0.1), fa.FA2_ERR_STRIDE),                            # FP8 rows of 72 bytes
    (dict(strides=_with(_SKV_CONTIG, s10=0, s9=0), H=2, B=2), fa.FA2_ERR_STRIDE),  # o rows shared
    (dict(strides=_with(_SKV_CONTIG, s5=1 << 23)), fa.FA2_ERR_SHAPE),   # 256 K rows span 2^32 B
    (dict(kv_fp8=1, k_descale=0.0), fa.FA2_ERR_SCALE),
    (dict(o=KS + 64), fa.FA2_ERR_ALIAS),
])
def test_splitkv_strided_validation_status(lib, kw, status):
    assert _call_splitkv_strided(**kw) == status


@pytest.mark.parametrize("kw", [
    dict(),
    dict(kv_fp8=1, k_descale=0.01, v_descale=0.02),
    # a cache of 4 * Sk rows read up to Sk, (B, S, H, D)-style head stride D
    dict(strides=_with(_SKV_CONTIG, s3=4 * _SK * _D, s4=_D, s5=2 * _D, s6=4 * _SK * _D, s7=_D,
                       s8=2 * _D), H=2),
], ids=["contiguous", "fp8", "cache_view"])
def test_splitkv_strided_valid_calls_reach_the_device_check(lib, kw):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    if kw.get("H") == 2:
        # two heads: o and lse grow, the workspace too
        kw = dict(kw, workspace_bytes=fa.fa2_splitkv_workspace_bytes(1, 2, _SQ, _SK, _D, 4),
                  strides=[2 * _SQ * _D, _SQ * _D, _D] + kw["strides"][3:9]
                  + [2 * _SQ * _D, _SQ * _D, _D])
    assert _call_splitkv_strided(**kw) == fa.FA2_ERR_NO_DEVICE


def test_splitkv_no_device_status_without_gpu(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the fake pointers must not be launched on")
    assert _call_splitkv() == fa.FA2_ERR_NO_DEVICE
    assert _call_splitkv(n_split=0) == fa.FA2_ERR_NO_DEVICE


def test_attention_splitkv_wrapper_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 2, 64, dtype=torch.float16)
    kv = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention_splitkv(q, kv, kv)  # CPU tensors
    with pytest.raises(ValueError):
        fa.attention_splitkv(q, kv, kv[:, :, :4])


# ---------------------------------------------------------------------------
# the matrix-core ceiling probe (include/fa2_probe.h, libfa2probe.so): a
# measurement aid of its own library, not part of the attention ABI
# ---------------------------------------------------------------------------
PROBE_HEADER = os.path.join(ROOT, "include", "fa2_probe.h")


def test_every_header_has_its_library():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["fa2.h", "fa2_probe.h", "fa2_timeline.h"]


@pytest.fixture(scope="module")
def probe():
    from flashattention_tiled_amd.build import PROBE_LIB_PATH, build_probe

    if not os.path.exists(PROBE_LIB_PATH):
        build_probe(force=False)
    import torch  # noqa: F401  (shares torch's HIP runtime)

    p = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    p.fa2_probe_mfma_ceiling.argtypes = [vp, i, i, vp, vp, i, vp]
    p.fa2_probe_mfma_ceiling.restype = i
    p.fa2_probe_mfma_flops.argtypes = [i, i]
    p.fa2_probe_mfma_flops.restype = ctypes.c_double
    p.fa2_probe_mfma_fp8.argtypes = [vp, vp, vp, vp, i, vp]
    p.fa2_probe_mfma_fp8.restype = i
    p.fa2_probe_cvt_fp8.argtypes = [vp, vp, i, vp]
    p.fa2_probe_cvt_fp8.restype = i
    return p


def test_cvt_probe_validates_before_launch(probe):
    A, B = 0x10000000, 0x10010000
    assert probe.fa2_probe_cvt_fp8(None, B, 4, None) == 1
    assert probe.fa2_probe_cvt_fp8(A, B, 6, None) == 2
    assert probe.fa2_probe_cvt_fp8(A, B, 0, None) == 2
    assert probe.fa2_probe_cvt_fp8(A + 4, B, 4, None) == 16


def test_fp8_probe_validates_before_launch(probe):
    A, B, C, D = 0x10000000, 0x10010000, 0x10020000, 0x10030000
    assert probe.fa2_probe_mfma_fp8(None, B, C, D, 1, None) == 1
    assert probe.fa2_probe_mfma_fp8(A, B, C, None, 1, None) == 1
    assert probe.fa2_probe_mfma_fp8(A, B, C, D, 0, None) == 2
    assert probe.fa2_probe_mfma_fp8(A + 16, B, C, D, 1, None) == 16
    assert probe.fa2_probe_mfma_fp8(A, B, C + 2, D, 1, None) == 16


def test_probe_exports_exactly_its_header(probe):
    from flashattention_tiled_amd.build import PROBE_LIB_PATH

    text = open(PROBE_HEADER).read()
    declared = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa2_\w+)\s*\(", text, flags=re.M)
    assert sorted(declared) == ["fa2_probe_cvt_fp8", "fa2_probe_mfma_ceiling",
                                "fa2_probe_mfma_flops", "fa2_probe_mfma_fp8"]
    _, defined = _elf_dynamic(PROBE_LIB_PATH)
    assert sorted(n for n in defined if n.startswith("fa2")) == sorted(declared)
    for name in declared:
        assert ctypes.cast(getattr(probe, name), ctypes.c_void_p).value


def test_probe_flops_and_validation(probe):
    # 4 waves x iters rounds x 16 products of 32 x 32 x 16 x 2 FLOPs per workgroup
    assert probe.fa2_probe_mfma_flops(3, 5) == 3 * 4 * 5 * 16 * 32 * 32 * 16 * 2
    fake = 1 << 20  # never dereferenced: validation returns first
    assert probe.fa2_probe_mfma_ceiling(None, 1, 1, fake, fake, 0, None) == 1
    assert probe.fa2_probe_mfma_ceiling(fake, 1, 1, None, fake, 0, None) == 1
    assert probe.fa2_probe_mfma_ceiling(fake, 1, 1, fake, None, 0, None) == 1
    assert probe.fa2_probe_mfma_ceiling(fake, 0, 1, fake, fake, 0, None) == 2
    assert probe.fa2_probe_mfma_ceiling(fake, 1, 0, fake, fake, 1, None) == 2
    assert probe.fa2_probe_mfma_ceiling(fake, 1, 1, fake, fake, 2, None) == 4
    assert probe.fa2_probe_mfma_ceiling(fake, 1, 1, fake, fake, -1, None) == 4


# ---------------------------------------------------------------------------
# the timeline build (include/fa2_timeline.h, libfa2_timeline.so): the same
# sources with per-workgroup clock stamps, a measurement aid of its own library
# ---------------------------------------------------------------------------
TIMELINE_HEADER = os.path.join(ROOT, "include", "fa2_timeline.h")


@pytest.fixture(scope="module")
def timeline():
    from flashattention_tiled_amd.build import TIMELINE_LIB_PATH, build_timeline

    if not os.path.exists(TIMELINE_LIB_PATH):
        build_timeline(force=False)
    import torch  # noqa: F401  (shares torch's HIP runtime)

    t = ctypes.CDLL(TIMELINE_LIB_PATH)
    t.fa2_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    return t


def test_timeline_exports_the_library_and_its_header(timeline):
    from flashattention_tiled_amd.build import TIMELINE_LIB_PATH

    text = open(TIMELINE_HEADER).read()
    declared = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa2_\w+)\s*\(", text, flags=re.M)
    assert sorted(declared) == ["fa2_timeline_capacity", "fa2_timeline_clear", "fa2_timeline_read"]
    _, defined = _elf_dynamic(TIMELINE_LIB_PATH)
    assert sorted(n for n in defined if n.startswith("fa2")) == sorted(declared + _declared_functions())
    # the product library records nothing and exports none of it
    _, product = _elf_dynamic(fa.LIB_PATH)
    assert not [n for n in product if "timeline" in n]


def test_timeline_read_validates_before_touching_the_device(timeline):
    cap = timeline.fa2_timeline_capacity()
    assert cap == 16384
    buf = (ctypes.c_ulonglong * 8)()
    assert timeline.fa2_timeline_read(None, 1) == fa.FA2_ERR_SHAPE
    assert timeline.fa2_timeline_read(ctypes.addressof(buf), -1) == fa.FA2_ERR_SHAPE
    assert timeline.fa2_timeline_read(ctypes.addressof(buf), cap + 1) == fa.FA2_ERR_SHAPE
