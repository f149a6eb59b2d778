"""Parity of the key-split forward (fa_fwd_split) with the CPU fp64 oracle.

Each head's keys are cut into ranges of whole 64-key tiles; the fused kernel computes
every range's (O_g, LSE_g) and a merge kernel combines them with the block-merge rule
(Triton tutorial section 2.3).  The result is the full attention, so it is held to the
same bar as fa_fwd: max |O - O_ref| <= 1e-2 and cosine >= 0.999 for 16-bit inputs,
<= 1e-5 for fp32 inputs, LSE within 1e-4 relative.
"""
import math

import numpy as np
import pytest

import oracle
from synth.configs import WORKLOADS
from synth.inputs import make_qkv
from tests.gpu_util import assert_parity, metrics, sample_rows, say, to_device

pytestmark = pytest.mark.gpu


def run_split(xd, scale, nsplit):
    import torch

    import exact_attention_90_amd as fa

    o, lse = fa.fwd_split(xd["q"], xd["k"], xd["v"], nsplit, scale)
    torch.cuda.synchronize()
    return o, lse


def split_case(B, H, N, d, dtype, nsplit, seed, mult=1.0):
    scale32 = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed, mult)
    say(f"split B={B} H={H} N={N} d={d} {dtype} nsplit={nsplit} seed={seed} mult={mult}")
    o, lse = run_split(to_device(x, dtype), scale32, nsplit)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], dtype, scale32)
    return metrics(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("B,H,N,d,dtype,nsplit", [
    (1, 2, 1000, 128, "bf16", 4),    # ragged last range and tile
    (1, 2, 1000, 128, "f16", 3),
    (2, 1, 333, 64, "f16", 2),
    (1, 1, 517, 256, "bf16", 5),
    (1, 2, 130, 128, "bf16", 8),     # more ranges than key tiles: three run
    (1, 1, 64, 128, "f16", 2),       # one key tile: one range runs
    (1, 3, 1, 64, "bf16", 4),        # one key
    (1, 1, 4096, 64, "f16", 64),     # the largest split, one tile per range
    (1, 2, 300, 128, "f32", 3),      # fp32 inputs (fp32 matrix cores)
    (1, 1, 200, 256, "f32", 2),      # fp32 at d = 256 (32-key tiles)
    (2, 1, 129, 64, "f32", 4),
])
def test_split_small_full(B, H, N, d, dtype, nsplit):
    m = split_case(B, H, N, d, dtype, nsplit, seed=N + d + nsplit)
    assert_parity(m, dtype, where=f"{B}x{H}x{N}x{d} {dtype} nsplit={nsplit}")


@pytest.mark.parametrize("dtype,mult", [("bf16", 3.0), ("f16", 8.0)])
def test_split_large_logits(dtype, mult):
    # ranges whose maxima differ widely: the merge weights exp(LSE_g - LSE) span many
    # orders of magnitude
    m = split_case(1, 2, 2048, 128, dtype, 4, seed=77, mult=mult)
    assert_parity(m, dtype, where=f"mult={mult}")


def test_split_one_range_is_bitwise_fa_fwd():
    import torch

    import exact_attention_90_amd as fa

    B, H, N, d = 2, 3, 700, 128
    xd = to_device(make_qkv(B, H, N, d, "bf16", seed=3), "bf16")
    say("nsplit=1 against fa_fwd")
    o1, l1 = run_split(xd, 1.0 / math.sqrt(d), 1)
    o0, l0 = fa.fwd(xd["q"], xd["k"], xd["v"], 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_split_bitwise_deterministic():
    import torch

    xd = to_device(make_qkv(1, 4, 3000, 128, "f16", seed=9), "f16")
    say("split determinism")
    outs = [run_split(xd, 1.0 / math.sqrt(128), 6) for _ in range(3)]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_split_long_sequence_few_heads_sampled():
    # the long-sequence workload (bf16 1x16x16384x128, inputs x3) through four key ranges
    w = WORKLOADS["c5"]
    scale32 = float(np.float32(w.scale))
    say(f"c5 split: generating {w.short()}")
    x = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    say("c5 split: fa_fwd_split nsplit=4")
    o, lse = run_split(to_device(x, w.dtype), scale32, 4)
    rows = sample_rows(w.B, w.H, w.N)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], w.dtype, scale32, rows=rows)
    import torch

    idx = torch.from_numpy(rows).to(o.device)
    o_s = o.reshape(-1, w.d).index_select(0, idx).cpu().numpy()
    l_s = lse.reshape(-1).index_select(0, idx).cpu().numpy()
    m = metrics(o_s, l_s, o_ref, lse_ref)
    say(f"c5 split: {m}")
    assert_parity(m, w.dtype, where="c5 split")
    assert bool(np.isfinite(o.cpu().numpy()).all())


def test_split_default_count_from_the_device():
    import exact_attention_90_amd as fa
    import torch

    B, H, N, d, dtype = 1, 1, 2048, 128, "bf16"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"default split count: {fa.split_suggest(B, H, N, d, cus)} of {cus} compute units")
    x = make_qkv(B, H, N, d, dtype, seed=8)
    scale32 = float(np.float32(1.0 / math.sqrt(d)))
    xd = to_device(x, dtype)
    o, lse = fa.fwd_split(xd["q"], xd["k"], xd["v"], scale=scale32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], dtype, scale32)
    assert_parity(metrics(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref), dtype,
                  where="default split")
