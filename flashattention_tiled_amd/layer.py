"""An attention layer around the FlashAttention-2 forward pass.

FA2Attention is the layer of the cookbook notebook "FlashAttention-2 in an
attention layer" ("Attention layer using the kernel"): a bias-free QKV
projection, the FA2 kernel in place of QK^T / softmax / AV, and a bias-free
output projection, causal by default. The projections are plain torch
Linear layers; the attention between them runs in libfa2.so.

Where the notebook transposes Q, K and V to (B, H, T, D) and copies them
contiguous before its kernel, this layer hands the kernel the strided
(B, H, T, D) views of the packed (B, T, 3, H, D) projection output
(fa2_fwd_strided) and lets it write O straight into a (B, T, H, D) buffer,
which the output projection reads as (B, T, H*D) without a copy.

The library has no backward pass, so the layer is for inference: calling it
where autograd would record it raises.

For generation the layer keeps keys and values in a KVCache (16-bit, or FP8
e4m3 codes with one descale per tensor): forward(x, cache) appends the new
tokens' K and V and attends their queries to the whole cache, causally with
the new tokens last, through the split-KV (FlashDecoding) path, which reads
the cache's buffers in place up to their current length.
"""
from __future__ import annotations

import torch
from torch import nn

from . import attention, attention_splitkv


class KVCache:
    """Keys and values of one attention layer for up to `max_len` tokens:
    (B, H, max_len, D) buffers filled up to `length`. fp8=True stores OCP
    e4m3 codes of value / descale (torch's round-to-nearest cast, saturated
    at 448); otherwise values in `dtype`."""

    def __init__(self, B: int, H: int, max_len: int, D: int, dtype=torch.float16, device=None,
                 fp8: bool = False, k_descale: float = 1.0, v_descale: float = 1.0):
        store = torch.float8_e4m3fn if fp8 else dtype
        self.k = torch.zeros((B, H, max_len, D), dtype=torch.uint8 if fp8 else dtype,
                             device=device).view(store)
        self.v = torch.zeros((B, H, max_len, D), dtype=torch.uint8 if fp8 else dtype,
                             device=device).view(store)
        self.fp8 = fp8
        self.k_descale, self.v_descale = float(k_descale), float(v_descale)
        self.length = 0

    def append(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """Add (B, H, T, D) keys and values after the cached ones."""
        T = k.shape[2]
        if self.length + T > self.k.shape[2]:
            raise ValueError(f"the cache holds {self.k.shape[2]} tokens; "
                             f"{self.length} + {T} do not fit")
        end = self.length + T
        if self.fp8:
            k = (k.float() / self.k_descale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            v = (v.float() / self.v_descale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        self.k[:, :, self.length:end] = k
        self.v[:, :, self.length:end] = v
        self.length = end

    def view(self):
        """The cached keys and values, (B, H, length, D) views of the buffers."""
        return self.k[:, :, :self.length], self.v[:, :, :self.length]


class FA2Attention(nn.Module):
    """Self-attention: x (B, T, d_model) -> (B, T, d_model) with num_heads
    heads of d_model // num_heads dims (64, 128 or 256), fp16 or bf16."""

    def __init__(self, d_model: int, num_heads: int, causal: bool = True, device=None,
                 dtype=None) -> None:
        super().__init__()
        if d_model % num_heads:
            raise ValueError("d_model must be a multiple of num_heads")
        self.num_heads = num_heads
        self.head_dim = d_model // num_heads
        self.causal = causal
        self.qkv = nn.Linear(d_model, 3 * d_model, bias=False, device=device, dtype=dtype)
        self.o = nn.Linear(d_model, d_model, bias=False, device=device, dtype=dtype)

    def attend(self, qkv: torch.Tensor) -> torch.Tensor:
        """The attention step alone: qkv (B, T, 3 * d_model) from the QKV
        projection -> (B, T, d_model), the input of the output projection."""
        B, T, _ = qkv.shape
        H, D = self.num_heads, self.head_dim
        q, k, v = qkv.view(B, T, 3, H, D).unbind(dim=2)  # (B, T, H, D) views
        out = torch.empty((B, T, H, D), dtype=qkv.dtype, device=qkv.device)
        attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), causal=self.causal,
                  out=out.transpose(1, 2))
        return out.view(B, T, H * D)

    def attend_cached(self, qkv: torch.Tensor, cache: KVCache) -> torch.Tensor:
        """The attention step with a cache: append the new tokens' K and V
        from qkv (B, T, 3 * d_model), then attend their queries to every
        cached token (causal: the new tokens are the last T). Returns
        (B, T, d_model). A 16-bit cache that held nothing before runs the
        prefill kernel on it; otherwise the split-KV path reads the cache."""
        B, T, _ = qkv.shape
        H, D = self.num_heads, self.head_dim
        q, k, v = (t.transpose(1, 2) for t in qkv.view(B, T, 3, H, D).unbind(dim=2))
        first = cache.length == 0
        cache.append(k, v)
        kc, vc = cache.view()
        out = torch.empty((B, T, H, D), dtype=qkv.dtype, device=qkv.device)
        if first and not cache.fp8:
            attention(q, kc, vc, causal=self.causal, out=out.transpose(1, 2))
        else:
            attention_splitkv(q, kc, vc, causal=self.causal, out=out.transpose(1, 2),
                              k_descale=cache.k_descale, v_descale=cache.v_descale)
        return out.view(B, T, H * D)

    def forward(self, x: torch.Tensor, cache: KVCache | None = None) -> torch.Tensor:
        if torch.is_grad_enabled() and (x.requires_grad or
                                        any(p.requires_grad for p in self.parameters())):
            raise RuntimeError("FA2Attention has no backward pass: call it under "
                               "torch.inference_mode() or torch.no_grad()")
        if cache is None:
            return self.o(self.attend(self.qkv(x)))
        return self.o(self.attend_cached(self.qkv(x), cache))
