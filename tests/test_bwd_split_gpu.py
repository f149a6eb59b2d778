"""Parity of the split backward pass (fa_bwd_split) with the CPU fp64 oracle.

The key-owned kernel's query tiles and the query-owned kernel's key tiles are cut into
ranges; each range's partial dQ, dK, dV goes to its own slot and the slots are added in
order.  The gradients are the same sums, regrouped, so the bar is fa_bwd's (rms_rel <=
3 u, max_rel <= 12 u against the oracle's gradients; see test_bwd_gpu.py).
"""
import math

import numpy as np
import pytest

import oracle
from synth.inputs import make_dout, make_qkv
from tests.gpu_util import say, to_device
from tests.test_bwd_gpu import assert_grads

pytestmark = pytest.mark.gpu


def run(x, g_np, dtype, scale, nsplit):
    import torch

    import exact_attention_90_amd as fa

    xd = to_device(x, dtype)
    o, lse = fa.fwd(xd["q"], xd["k"], xd["v"], scale)
    g = torch.from_numpy(g_np).to("cuda")
    split = fa.bwd_split(xd["q"], xd["k"], xd["v"], o, lse, g, nsplit, scale)
    torch.cuda.synchronize()
    return xd, o, lse, g, split


@pytest.mark.parametrize("B,H,N,d,dtype,nsplit", [
    (1, 2, 300, 128, "bf16", 3),     # ragged last range and tile
    (1, 1, 700, 64, "f16", 4),
    (1, 1, 333, 256, "bf16", 2),     # d = 256: dV and dK in two launches, both split
    (2, 1, 129, 128, "f16", 8),      # more ranges than tiles: three run
    (1, 1, 64, 64, "bf16", 2),       # one tile: one range runs
    (1, 1, 300, 64, "f32", 3),       # fp32 inputs (fp32 matrix cores)
    (1, 2, 200, 128, "f32", 2),
])
def test_bwd_split_small_full(B, H, N, d, dtype, nsplit):
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed=N + d + nsplit)
    g = make_dout(B, H, N, d, seed=N + 7)
    say(f"bwd_split B={B} H={H} N={N} d={d} {dtype} nsplit={nsplit}")
    _, _, _, _, split = run(x, g, dtype, scale, nsplit)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, scale)
    assert_grads([t.cpu().numpy() for t in split], ref, dtype,
                 f"{B}x{H}x{N}x{d} {dtype} nsplit={nsplit}")


def test_bwd_split_one_range_is_bitwise_fa_bwd():
    import torch

    import exact_attention_90_amd as fa

    B, H, N, d, dtype = 1, 2, 500, 128, "bf16"
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed=4)
    g = make_dout(B, H, N, d, seed=5)
    say("bwd_split nsplit=1 against fa_bwd")
    xd, o, lse, gt, split = run(x, g, dtype, scale, 1)
    full = fa.bwd(xd["q"], xd["k"], xd["v"], o, lse, gt, scale)
    torch.cuda.synchronize()
    for a, b in zip(split, full):
        assert torch.equal(a, b)


def test_bwd_split_deterministic():
    import torch

    import exact_attention_90_amd as fa

    B, H, N, d, dtype = 1, 1, 1500, 64, "f16"
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed=6)
    g = make_dout(B, H, N, d, seed=7)
    say("bwd_split determinism")
    xd, o, lse, gt, first = run(x, g, dtype, scale, 5)
    for _ in range(2):
        again = fa.bwd_split(xd["q"], xd["k"], xd["v"], o, lse, gt, 5, scale)
        torch.cuda.synchronize()
        for a, b in zip(again, first):
            assert torch.equal(a, b)


def test_bwd_split_one_long_head():
    # one head of 4096 rows (32 workgroups per kernel without a split), default count
    B, H, N, d, dtype = 1, 1, 4096, 128, "bf16"
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed=11)
    g = make_dout(B, H, N, d, seed=12)
    say("bwd_split one head N=4096, default count")
    _, _, _, _, split = run(x, g, dtype, scale, None)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, scale)
    assert_grads([t.cpu().numpy() for t in split], ref, dtype, "one head N=4096")
