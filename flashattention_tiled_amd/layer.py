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
"""
from __future__ import annotations

import torch
from torch import nn

from . import attention


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

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if torch.is_grad_enabled() and (x.requires_grad or
                                        any(p.requires_grad for p in self.parameters())):
            raise RuntimeError("FA2Attention has no backward pass: call it under "
                               "torch.inference_mode() or torch.no_grad()")
        return self.o(self.attend(self.qkv(x)))
