"""The D = 128 and D = 64 tiles that split each query tile's keys between
two wave groups (merged through LDS), against the fp64 oracle on every output.

fa2_fwd takes them for causal grids whose main-tile workgroups are all
resident at once with at least one per compute unit (256 to 512 query tiles
of 128 rows on the 256 units of an MI355X; D = 64 below its long-sequence
tile's S). The cases cover the split at
every query tile, including the first (whose keys all go to the second
group), ragged sequence ends inside a group's last tile, an odd number of
key tiles (the groups run different numbers of tiles), both dtypes, a
negative scale, strided views, grids from one to two tiles per compute unit
(the LLM layer's among them), and the shape beside it that keeps the main
tile. Tolerances: max |dO| <= 2e-3 (fp16) / 1.6e-2 (bf16), lse relative
error <= 1e-4.
"""
import math

import pytest
import torch

import flashattention_tiled_amd as fa
import workloads as wl
from gpu_helpers import DEV, announce, assert_parity, oracle_full

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, S, dtype, scale sign[, D]): query tiles = ceil(S / 128) * B * H
    (1, 40, 1000, "f16", 1),     # 320 tiles, ragged end inside a key tile
    (2, 8, 4000, "bf16", 1),     # 512 tiles, 63 key tiles per long row block
    (1, 4, 8192, "f16", 1),      # 256 tiles: one long head per 64 units
    (1, 36, 960, "f16", -1),     # 288 tiles, negative scale
    (1, 16, 2049, "bf16", 1),    # 272 tiles, a one-row last tile
    (1, 32, 2048, "f16", 1),     # 512 tiles: the LLM layer's attention
    (1, 30, 1900, "bf16", 1),    # 450 tiles, 15 per head, ragged end
    (2, 16, 1700, "f16", -1),    # 448 tiles, 14 per head, ragged end, negative scale
    (2, 16, 1024, "f16", 1, 64),    # D = 64: 256 tiles
    (1, 32, 2048, "bf16", 1, 64),   # D = 64: 512 tiles
    (1, 20, 1700, "f16", -1, 64),   # D = 64: 280 tiles, ragged end, negative scale
    (1, 16, 4097, "bf16", 1, 64),   # D = 64: 528 > 512 tiles, the main tile beside it
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_key_groups_every_row(case):
    B, H, S, dt, sign = case[:5]
    D = case[5] if len(case) > 5 else 128
    w = wl.Workload("key_groups", B, H, S, D, dt, True)
    scale = sign / math.sqrt(D)
    announce(f"key groups B={B} H={H} S={S} D={D} {dt} scale={scale:+.4f}")
    q, k, v = wl.make_qkv(w, seed=S + H)
    # fa2_fwd itself (attention() may take the key split of fa2_fwd_balanced)
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale,
                          balanced=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, True, scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, dt, f"key groups {case}")


def test_key_groups_q_rows_apart_from_kv():
    """Q as a (B, S, H, D) view (rows H * D apart) beside K and V whose rows
    are padded to D + 64: Q's half tiles go through LDS with Q's own stride."""
    B, H, S, D = 1, 40, 1000, 128
    announce(f"key groups Q stride apart B={B} H={H} S={S}")
    w = wl.Workload("key_groups_mixed", B, H, S, D, "bf16", True)
    q, k, v = wl.make_qkv(w, seed=9)
    q_view = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    kv = []
    for x in (k, v):
        buf = torch.full((B, H, S, D + 64), float("nan"), dtype=x.dtype)
        buf[..., :D] = x
        kv.append(buf.to(DEV)[..., :D])
    o, lse = fa.attention(q_view, kv[0], kv[1], causal=True, scale=w.scale, balanced=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, True, w.scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, "bf16", "key groups Q stride apart")


@pytest.mark.parametrize("D", [128, 64])
def test_key_groups_strided(D):
    """Q, K and V as views into one packed (B, S, 3, H, D) projection."""
    B, H, S = 1, 48, 700
    announce(f"key groups strided B={B} H={H} S={S} D={D}")
    w = wl.Workload("key_groups_strided", B, H, S, D, "f16", True)
    q, k, v = wl.make_qkv(w, seed=7)
    packed = torch.empty((B, S, 3, H, D), dtype=torch.float16, device=DEV)
    packed[:, :, 0] = q.permute(0, 2, 1, 3).to(DEV)
    packed[:, :, 1] = k.permute(0, 2, 1, 3).to(DEV)
    packed[:, :, 2] = v.permute(0, 2, 1, 3).to(DEV)
    qs, ks, vs = (packed[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    o, lse = fa.attention(qs, ks, vs, causal=True, scale=w.scale, balanced=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, True, w.scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, "f16", "key groups strided")
