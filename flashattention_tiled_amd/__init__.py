"""FlashAttention-2 forward pass for MI355X (gfx950): thin Python binding.

Every step of the forward pass runs in the HIP library ``libfa2.so`` built
from ``csrc/``; this module only marshals arguments to its C ABI
(declared in ``include/fa2.h``). PyTorch is used for device memory and
streams. There is no fallback: if the library is missing, importing the
binding's functions raises.

C entry points, re-exported under the same names:
    fa2_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, stream) -> int
    fa2_fwd_strided(q, k, v, o, lse, B, H, S, D, strides, causal, scale, dtype,
                    stream) -> int   (strides: 12 element strides)
    fa2_fwd_balanced(q, k, v, o, lse, B, H, S, D, strides, causal, scale, dtype,
                     workspace, workspace_bytes, stream) -> int   (strides or None)
    fa2_fwd_balanced_workspace_bytes(B, H, S, D, causal) -> int
    fa2_supported(D, dtype) -> int
    fa2_status_string(status) -> str
    fa2_rows_per_workgroup(D) -> int
    fa2_fwd_splitkv(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, dtype,
                    n_split, workspace, workspace_bytes, stream) -> int
    fa2_fwd_splitkv_fp8(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale,
                        k_descale, v_descale, dtype, n_split, workspace,
                        workspace_bytes, stream) -> int
    fa2_fwd_splitkv_strided(q, k, v, o, lse, B, H, Sq, Sk, D, strides, causal,
                            scale, dtype, kv_fp8, k_descale, v_descale, n_split,
                            workspace, workspace_bytes, stream) -> int
    fa2_fwd_fp8(q, k, v, o, lse, B, H, S, D, causal, scale, q_descale, k_descale,
                v_descale, dtype, stream) -> int   (e4m3 q, k, v; fp16/bf16 o)
    fa2_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, dtype,
                            n_split, stream) -> int   (no workspace, allocates nothing)
    fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n_split) -> int
    fa2_splitkv_splits(B, H, Sq, Sk) -> int
    fa2_splitkv_splits_fp8(B, H, Sq, Sk) -> int
plus the tensor-level conveniences ``attention(q, k, v, causal, scale)`` (any
layout whose head dim is contiguous; the key-split fa2_fwd_balanced when the
library plans a split for the shape) and
``attention_splitkv(q, k, v, causal, scale, n_split)`` (Sq queries against Sk
cached keys).
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")

# fa2_dtype
FA2_F16 = 0
FA2_BF16 = 1

# fa2_status
FA2_OK = 0
FA2_ERR_NULL = 1
FA2_ERR_SHAPE = 2
FA2_ERR_HEADDIM = 3
FA2_ERR_DTYPE = 4
FA2_ERR_ALIGN = 5
FA2_ERR_SCALE = 6
FA2_ERR_NO_DEVICE = 7
FA2_ERR_LAUNCH = 8
FA2_ERR_ALIAS = 9
FA2_ERR_WORKSPACE = 10
FA2_ERR_STRIDE = 11
FA2_ERR_SCRATCH = 12

EXPORTED_SYMBOLS = ("fa2_fwd", "fa2_fwd_strided", "fa2_fwd_balanced",
                    "fa2_fwd_balanced_workspace_bytes", "fa2_supported", "fa2_status_string",
                    "fa2_rows_per_workgroup", "fa2_fwd_splitkv", "fa2_fwd_splitkv_fp8",
                    "fa2_fwd_splitkv_strided", "fa2_fwd_splitkv_noalloc", "fa2_fwd_fp8",
                    "fa2_splitkv_workspace_bytes", "fa2_splitkv_splits",
                    "fa2_splitkv_splits_fp8")


class FA2Error(RuntimeError):
    """A nonzero fa2_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"fa2 status {status}: {message}")
        self.status = status


_lib = None


def _hip_runtimes_mapped() -> list:
    """Paths of the HIP runtime libraries (libamdhip64) mapped into this
    process (Linux), one per copy."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa2.so (once). Raises OSError when it has not been built.

    The library must share torch's HIP runtime: the device pointers and
    streams it is given come from torch. torch ships its own libamdhip64 with
    the same soname as the system one, so torch is imported first and the
    library's dependency then resolves to torch's copy. Loading it before
    torch would map a second HIP runtime, on which torch's device and
    allocations do not exist; that case raises instead of running."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with flashattention_tiled_amd.build "
                      f"(or __graft_entry__.build()) before use")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)

    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise OSError("two HIP runtimes are loaded in this process (" + ", ".join(runtimes) +
                      "); libfa2.so must share torch's: import torch before loading any "
                      "other library that links libamdhip64")
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa2_fwd.restype = i
    lib.fa2_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i,
                                    ctypes.POINTER(ctypes.c_longlong), i, f, i, vp]
    lib.fa2_fwd_strided.restype = i
    sz = ctypes.c_size_t
    lib.fa2_fwd_balanced.argtypes = [vp, vp, vp, vp, vp, i, i, i, i,
                                     ctypes.POINTER(ctypes.c_longlong), i, f, i, vp, sz, vp]
    lib.fa2_fwd_balanced.restype = i
    lib.fa2_fwd_balanced_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa2_fwd_balanced_workspace_bytes.restype = sz
    lib.fa2_supported.argtypes = [i, i]
    lib.fa2_supported.restype = i
    lib.fa2_status_string.argtypes = [i]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_rows_per_workgroup.argtypes = [i]
    lib.fa2_rows_per_workgroup.restype = i
    lib.fa2_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa2_fwd_splitkv.restype = i
    lib.fa2_fwd_splitkv_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, i, i, vp, sz,
                                        vp]
    lib.fa2_fwd_splitkv_fp8.restype = i
    lib.fa2_fwd_splitkv_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i,
                                            ctypes.POINTER(ctypes.c_longlong), i, f, i, i, f, f,
                                            i, vp, sz, vp]
    lib.fa2_fwd_splitkv_strided.restype = i
    lib.fa2_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, i, vp]
    lib.fa2_fwd_fp8.restype = i
    lib.fa2_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa2_fwd_splitkv_noalloc.restype = i
    lib.fa2_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa2_splitkv_workspace_bytes.restype = sz
    lib.fa2_splitkv_splits.argtypes = [i, i, i, i]
    lib.fa2_splitkv_splits.restype = i
    lib.fa2_splitkv_splits_fp8.argtypes = [i, i, i, i]
    lib.fa2_splitkv_splits_fp8.restype = i
    _lib = lib
    return lib


def fa2_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
            causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(load_library().fa2_fwd(q, k, v, o, lse, B, H, S, D, int(causal),
                                      float(scale), int(dtype), stream))


def fa2_fwd_strided(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
                    strides, causal: int, scale: float, dtype: int, stream: int) -> int:
    """Direct call of the strided entry point; `strides` is a sequence of 12
    element strides (batch, head, seq of q, k, v, o). Returns the status."""
    st = None if strides is None else (ctypes.c_longlong * 12)(*[int(x) for x in strides])
    return int(load_library().fa2_fwd_strided(q, k, v, o, lse, B, H, S, D, st, int(causal),
                                              float(scale), int(dtype), stream))


def fa2_fwd_balanced(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
                     strides, causal: int, scale: float, dtype: int, workspace: int,
                     workspace_bytes: int, stream: int) -> int:
    """Direct call of the key-split entry point; `strides` is None
    (contiguous tensors) or 12 element strides. Returns the status."""
    st = None if strides is None else (ctypes.c_longlong * 12)(*[int(x) for x in strides])
    return int(load_library().fa2_fwd_balanced(q, k, v, o, lse, B, H, S, D, st, int(causal),
                                               float(scale), int(dtype), workspace,
                                               int(workspace_bytes), stream))


def fa2_fwd_balanced_workspace_bytes(B: int, H: int, S: int, D: int, causal: int) -> int:
    return int(load_library().fa2_fwd_balanced_workspace_bytes(B, H, S, D, int(causal)))


def fa2_supported(D: int, dtype: int) -> int:
    return int(load_library().fa2_supported(D, dtype))


def fa2_status_string(status: int) -> str:
    return load_library().fa2_status_string(status).decode()


def fa2_rows_per_workgroup(D: int) -> int:
    return int(load_library().fa2_rows_per_workgroup(D))


def fa2_fwd_splitkv(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Sk: int,
                    D: int, causal: int, scale: float, dtype: int, n_split: int, workspace: int,
                    workspace_bytes: int, stream: int) -> int:
    """Direct call of the split-KV C entry point with raw device addresses."""
    return int(load_library().fa2_fwd_splitkv(q, k, v, o, lse, B, H, Sq, Sk, D, int(causal),
                                              float(scale), int(dtype), int(n_split),
                                              workspace, int(workspace_bytes), stream))


def fa2_fwd_splitkv_fp8(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int,
                        Sk: int, D: int, causal: int, scale: float, k_descale: float,
                        v_descale: float, dtype: int, n_split: int, workspace: int,
                        workspace_bytes: int, stream: int) -> int:
    """Direct call of the FP8 K/V split-KV entry point; returns the status."""
    return int(load_library().fa2_fwd_splitkv_fp8(
        q, k, v, o, lse, B, H, Sq, Sk, D, int(causal), float(scale), float(k_descale),
        float(v_descale), int(dtype), int(n_split), workspace, int(workspace_bytes), stream))


def fa2_fwd_splitkv_strided(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int,
                            Sk: int, D: int, strides, causal: int, scale: float, dtype: int,
                            kv_fp8: int, k_descale: float, v_descale: float, n_split: int,
                            workspace: int, workspace_bytes: int, stream: int) -> int:
    """Direct call of the strided split-KV entry point; `strides` is a
    sequence of 12 element strides (batch, head, seq of q, k, v, o)."""
    st = None if strides is None else (ctypes.c_longlong * 12)(*[int(x) for x in strides])
    return int(load_library().fa2_fwd_splitkv_strided(
        q, k, v, o, lse, B, H, Sq, Sk, D, st, int(causal), float(scale), int(dtype), int(kv_fp8),
        float(k_descale), float(v_descale), int(n_split), workspace, int(workspace_bytes),
        stream))


def fa2_fwd_fp8(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
                causal: int, scale: float, q_descale: float, k_descale: float, v_descale: float,
                dtype: int, stream: int) -> int:
    """Direct call of the FP8 (e4m3 Q, K, V) prefill entry point; returns the status."""
    return int(load_library().fa2_fwd_fp8(q, k, v, o, lse, B, H, S, D, int(causal), float(scale),
                                          float(q_descale), float(k_descale), float(v_descale),
                                          int(dtype), stream))


def attention_fp8(q, k, v, causal: bool = False, scale: float | None = None,
                  q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0,
                  out_dtype=None, out=None, lse=None, stream=None):
    """O, lse of attention over FP8 inputs: q, k, v are contiguous (B, H, S,
    D) torch.float8_e4m3fn CUDA tensors whose values are codes times the
    descales; O is fp16 (default) or bf16 (`out_dtype`), lse (B, H, S)
    float32. Runs fa2_fwd_fp8 on `stream` (default: torch's current stream)
    without synchronising. Raises FA2Error on any nonzero status."""
    import torch

    fp8 = getattr(torch, "float8_e4m3fn", None)
    if fp8 is None or not (q.dtype == k.dtype == v.dtype == fp8):
        raise ValueError("q, k and v must be torch.float8_e4m3fn tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one (B, H, S, D) shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v must be contiguous")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or torch.float16
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty((B, H, S, D), dtype=out_dtype, device=q.device)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, S) tensor")
    with torch.cuda.device(q.device):
        status = fa2_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, S, D, int(bool(causal)), float(scale),
                             float(q_descale), float(k_descale), float(v_descale),
                             _dtype_code(out), stream.cuda_stream)
    if status != FA2_OK:
        raise FA2Error(status, fa2_status_string(status))
    return out, lse


def fa2_fwd_splitkv_noalloc(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int,
                            Sk: int, D: int, causal: int, scale: float, dtype: int, n_split: int,
                            stream: int) -> int:
    """Direct call of the split-KV entry point that allocates nothing (its
    partials go to the library's fixed scratch); returns the status."""
    return int(load_library().fa2_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D,
                                                      int(causal), float(scale), int(dtype),
                                                      int(n_split), stream))


def fa2_splitkv_workspace_bytes(B: int, H: int, Sq: int, Sk: int, D: int, n_split: int) -> int:
    return int(load_library().fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n_split))


def fa2_splitkv_splits_fp8(B: int, H: int, Sq: int, Sk: int) -> int:
    return int(load_library().fa2_splitkv_splits_fp8(B, H, Sq, Sk))


def fa2_splitkv_splits(B: int, H: int, Sq: int, Sk: int) -> int:
    return int(load_library().fa2_splitkv_splits(B, H, Sq, Sk))


def _dtype_code(t):
    import torch

    if t.dtype == torch.float16:
        return FA2_F16
    if t.dtype == torch.bfloat16:
        return FA2_BF16
    return -1


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
              stream=None, balanced: bool = True, workspace=None):
    """O, lse = softmax(scale * q k^T [causal]) v for (B, H, S, D) CUDA tensors.

    q, k, v: torch tensors on one GPU, fp16 or bf16, same shape, each with a
    contiguous last (head) dim; other strides are free (e.g. the (B, H, S, D)
    views of a packed (B, S, 3, H, D) projection). Contiguous tensors go to
    fa2_fwd, others to fa2_fwd_strided; with `balanced` (the default), shapes
    whose grid is too small to keep the GPU busy to the end go to
    fa2_fwd_balanced instead, with `workspace` (a CUDA uint8 tensor of at
    least fa2_fwd_balanced_workspace_bytes bytes) or one allocated with
    torch. scale defaults to 1/sqrt(D). Returns
    (o, lse): o of q's shape (a new contiguous tensor unless `out`, which may
    be any view with a contiguous last dim, is given), lse (B, H, S) float32
    (natural-log logsumexp per row). Runs on `stream` (default: torch's
    current stream) without synchronising. Raises FA2Error on any nonzero
    status.
    """
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one (B, H, S, D) shape, got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must have one dtype")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if not (q.stride(3) == 1 and k.stride(3) == 1 and v.stride(3) == 1):
        raise ValueError("q, k and v must have a contiguous last (head) dim")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    # Tensors made here are allocated on the launch stream: torch's caching
    # allocator then hands their memory to another allocation only in that
    # stream's order, after the kernels that use it.
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(3) != 1:
        raise ValueError("out must be a tensor of q's shape and dtype with a contiguous last dim")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, S) tensor")
    contiguous = all(t.is_contiguous() for t in (q, k, v, out))
    with torch.cuda.device(q.device):
        need = fa2_fwd_balanced_workspace_bytes(B, H, S, D, int(bool(causal))) if balanced else 0
        if need > 0:
            if workspace is None:
                with torch.cuda.stream(stream):
                    workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
            strides = None if contiguous else [x for t in (q, k, v, out) for x in t.stride()[:3]]
            status = fa2_fwd_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), B, H, S, D, strides, int(bool(causal)),
                                      float(scale), _dtype_code(q), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(),
                                      stream.cuda_stream)
        elif contiguous:
            status = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, S, D, int(bool(causal)), float(scale),
                             _dtype_code(q), stream.cuda_stream)
        else:
            strides = [x for t in (q, k, v, out) for x in t.stride()[:3]]
            status = fa2_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, H, S, D, strides, int(bool(causal)),
                                     float(scale), _dtype_code(q), stream.cuda_stream)
    if status != FA2_OK:
        raise FA2Error(status, fa2_status_string(status))
    return out, lse


def attention_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                      n_split: int = 0, out=None, lse=None, workspace=None, stream=None,
                      k_descale: float = 1.0, v_descale: float = 1.0):
    """O, lse for Sq queries against Sk cached keys: q (B, H, Sq, D), k and v
    (B, H, Sk, D), CUDA tensors with a contiguous last dim (other strides
    free: fa2_fwd_splitkv_strided). q is fp16 or bf16; k and v have
    q's dtype, or are both torch.float8_e4m3fn codes whose values are
    code * k_descale and code * v_descale (fa2_fwd_splitkv_fp8). Causal keeps
    key j for query i iff j <= i + Sk - Sq (the queries are the last Sq
    positions). n_split = 0 lets the library pick the number of key chunks.
    `workspace` may be passed preallocated (a CUDA uint8 tensor of at least
    fa2_splitkv_workspace_bytes bytes); otherwise one is allocated with torch.
    Returns (o like q, lse (B, H, Sq) float32). Raises FA2Error on any
    nonzero status.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError(f"q must be (B, H, Sq, D) and k, v (B, H, Sk, D), got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    fp8 = getattr(torch, "float8_e4m3fn", None)
    kv8 = fp8 is not None and k.dtype == fp8 and v.dtype == fp8
    if not (kv8 or q.dtype == k.dtype == v.dtype):
        raise ValueError("k and v must have q's dtype, or both be float8_e4m3fn")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    if not (q.stride(3) == 1 and k.stride(3) == 1 and v.stride(3) == 1):
        raise ValueError("q, k and v must have a contiguous last (head) dim")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    # allocated on the launch stream (see attention())
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(3) != 1:
        raise ValueError("out must be a tensor like q with a contiguous last dim")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, H, Sq) tensor")
    contiguous = all(t.is_contiguous() for t in (q, k, v, out))
    with torch.cuda.device(q.device):
        if n_split == 0:
            n_split = (fa2_splitkv_splits_fp8 if kv8 else fa2_splitkv_splits)(B, H, Sq, Sk)
        need = fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n_split)
        if workspace is None:
            with torch.cuda.stream(stream):
                workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        if not contiguous:
            strides = [x for t in (q, k, v, out) for x in t.stride()[:3]]
            status = fa2_fwd_splitkv_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                Sq, Sk, D, strides, int(bool(causal)), float(scale), _dtype_code(q), int(kv8),
                float(k_descale), float(v_descale), n_split, workspace.data_ptr(), ws_bytes,
                stream.cuda_stream)
        elif kv8:
            status = fa2_fwd_splitkv_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), B, H, Sq, Sk, D, int(bool(causal)),
                                         float(scale), float(k_descale), float(v_descale),
                                         _dtype_code(q), n_split, workspace.data_ptr(), ws_bytes,
                                         stream.cuda_stream)
        else:
            status = fa2_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, H, Sq, Sk, D, int(bool(causal)),
                                     float(scale), _dtype_code(q), n_split, workspace.data_ptr(),
                                     ws_bytes, stream.cuda_stream)
    if status != FA2_OK:
        raise FA2Error(status, fa2_status_string(status))
    return out, lse
