"""Parity of the HIP backward pass (fa_bwd) with the CPU fp64 oracle.

Bar, for each of dQ, dK, dV against the oracle's gradients (from the same storage
bits and the same float32 dO):
    rms_rel = ||X - X_ref||_2 / ||X_ref||_2      <= 3 u
    max_rel = max |X - X_ref| / max |X_ref|     <= 12 u
with u the unit roundoff of the input type (bf16 2^-8, fp16 2^-11).  Every product
runs on the matrix cores with two or three of its factors rounded to the input type
(dO, P, dS; round to nearest even, RMS relative error about 0.58 u each), so the
expected RMS relative error is about 1-1.5 u; the max over ~10^5 elements of such
errors stays below ~8 u.  For fp32 inputs nothing is rounded below fp32: u = 2^-16
covers fp32 rounding (2^-24) grown by sums of up to 4096 terms (x 2^6) and the
hardware exp2 (within 2 ulp, x 4).  The oracle's result is exact to double rounding.
"""
import math

import numpy as np
import pytest

import oracle
from synth.configs import HEADDIM_WORKLOADS, WORKLOADS
from synth.inputs import make_dout, make_qkv, quantize
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0**-8, "f16": 2.0**-11, "f32": 2.0**-16}


def run_bwd(x, dout, dtype, scale):
    import torch

    import exact_attention_90_amd as fa

    xd = to_device(x, dtype)
    o, lse = fa.fwd(xd["q"], xd["k"], xd["v"], scale)
    g = torch.from_numpy(dout).to("cuda")
    dq, dk, dv = fa.bwd(xd["q"], xd["k"], xd["v"], o, lse, g, scale)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def grad_metrics(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    err = got - ref
    return dict(rms_rel=float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)),
                max_rel=float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300)),
                finite=bool(np.isfinite(got).all()))


def assert_grads(gpu, ref, dtype, where):
    u = UNIT[dtype]
    for name, a, b in zip(("dq", "dk", "dv"), gpu, ref):
        m = grad_metrics(a, b)
        say(f"{where} {name}: {m}")
        assert m["finite"], f"{where} {name}: non-finite"
        assert m["rms_rel"] <= 3 * u, f"{where} {name}: rms_rel {m['rms_rel']:.3e} > {3 * u:.3e}"
        assert m["max_rel"] <= 12 * u, f"{where} {name}: max_rel {m['max_rel']:.3e} > {12 * u:.3e}"


def full_case(B, H, N, d, dtype, seed, mult=1.0):
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed, mult)
    g = make_dout(B, H, N, d, seed + 5000)
    say(f"bwd B={B} H={H} N={N} d={d} {dtype} seed={seed} mult={mult}")
    gpu = run_bwd(x, g, dtype, scale)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, scale)
    return gpu, ref


@pytest.mark.parametrize("B,H,N,d,dtype", [
    (1, 2, 128, 64, "bf16"), (1, 2, 128, 64, "f16"), (2, 2, 256, 128, "bf16"),
    (1, 3, 333, 128, "f16"), (1, 2, 200, 64, "bf16"), (2, 1, 1000, 128, "bf16"),
    (1, 2, 65, 128, "f16"), (1, 1, 700, 64, "f16"),
])
def test_bwd_small_full(B, H, N, d, dtype):
    gpu, ref = full_case(B, H, N, d, dtype, seed=N + d)
    assert_grads(gpu, ref, dtype, f"{B}x{H}x{N}x{d} {dtype}")


# key/query block counts 1..3 with ragged tails on both sides of each kernel's
# 128-row resident block and 64-row streamed tile
@pytest.mark.parametrize("N", [1, 2, 31, 64, 127, 129, 191, 257])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_bwd_lengths(N, dtype, d):
    gpu, ref = full_case(1, 2, N, d, dtype, seed=600 + N)
    if N == 1:
        # one key: P = 1 and dS = 0 in exact arithmetic, so dQ = dK = 0; on the GPU P is 1
        # to float32 rounding and dP - D is the difference of two float32 sums of the same
        # products, so dS is a rounding residue.  dV = dO (rounded to the input type).
        tiny = 1e-4 * np.abs(ref[2]).max()
        assert np.abs(gpu[0]).max() <= tiny and np.abs(gpu[1]).max() <= tiny
        m = grad_metrics(gpu[2], ref[2])
        assert m["rms_rel"] <= 3 * UNIT[dtype] and m["max_rel"] <= 12 * UNIT[dtype], m
        return
    assert_grads(gpu, ref, dtype, f"N={N} d={d} {dtype}")


@pytest.mark.parametrize("dtype,mult", [("bf16", 3.0), ("f16", 4.0)])
def test_bwd_large_logits(dtype, mult):
    gpu, ref = full_case(1, 2, 1000, 128, dtype, seed=91, mult=mult)
    assert_grads(gpu, ref, dtype, f"x{mult}")


def test_bwd_constant_v_gives_zero_dq_dk():
    # equal V rows: O does not depend on P, so dQ = dK = 0; the kernels see dP - D as
    # a difference of two roundings of one value, which stays at rounding level
    B, H, N, d, dtype = 1, 2, 300, 128, "bf16"
    x = make_qkv(B, H, N, d, dtype, seed=92)
    x["v"] = quantize(np.full((B, H, N, d), 0.75, np.float32), dtype)
    g = make_dout(B, H, N, d, 5092)
    say("bwd constant V")
    dq, dk, dv = run_bwd(x, g, dtype, 1.0 / math.sqrt(d))
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, 1.0 / math.sqrt(d))
    scale_q = np.abs(ref[2]).max()  # dV's size sets the scale of the rounding residue
    assert np.abs(dq).max() <= 12 * UNIT[dtype] * scale_q
    assert np.abs(dk).max() <= 12 * UNIT[dtype] * scale_q
    assert grad_metrics(dv, ref[2])["rms_rel"] <= 3 * UNIT[dtype]


def test_bwd_bitwise_deterministic():
    B, H, N, d, dtype = 1, 4, 777, 128, "bf16"
    x = make_qkv(B, H, N, d, dtype, seed=93)
    g = make_dout(B, H, N, d, 5093)
    say("bwd determinism")
    a = run_bwd(x, g, dtype, 1.0 / math.sqrt(d))
    b = run_bwd(x, g, dtype, 1.0 / math.sqrt(d))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# d = 256: dV and dK come from two launches of the key-owned kernel
@pytest.mark.parametrize("B,H,N,dtype", [(1, 2, 200, "bf16"), (2, 1, 333, "f16"),
                                         (1, 1, 1000, "bf16"), (1, 2, 1, "f16"),
                                         (1, 2, 129, "bf16")])
def test_bwd_d256(B, H, N, dtype):
    gpu, ref = full_case(B, H, N, 256, dtype, seed=N + 256)
    if N == 1:
        tiny = 1e-4 * np.abs(ref[2]).max()
        assert np.abs(gpu[0]).max() <= tiny and np.abs(gpu[1]).max() <= tiny
        return
    assert_grads(gpu, ref, dtype, f"{B}x{H}x{N}x256 {dtype}")


# fp32 inputs: fp32 matrix cores, nothing rounded below fp32
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 128, 64), (1, 2, 200, 128), (2, 1, 333, 64),
                                     (1, 1, 65, 128), (1, 2, 700, 128)])
def test_bwd_f32(B, H, N, d):
    gpu, ref = full_case(B, H, N, d, "f32", seed=N + d + 32)
    assert_grads(gpu, ref, "f32", f"{B}x{H}x{N}x{d} f32")


def test_bwd_larger_sampled_heads():
    # a larger problem: every gradient of two heads (first and last) against the oracle
    B, H, N, d, dtype = 2, 8, 2048, 128, "bf16"
    scale = float(np.float32(1.0 / math.sqrt(d)))
    x = make_qkv(B, H, N, d, dtype, seed=94)
    g = make_dout(B, H, N, d, 5094)
    say("bwd B2 H8 N2048 d128 bf16")
    gpu = run_bwd(x, g, dtype, scale)
    heads = [0, B * H - 1]
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, scale, heads=heads)
    sel = [a.reshape(B * H, N, d)[heads] for a in gpu]
    assert_grads(sel, ref, dtype, "B2H8N2048 heads 0,15")
    for a in gpu:
        assert np.isfinite(a).all()


@pytest.mark.parametrize("name", ["c3", "d256"])
def test_bwd_workload_full_size_sampled(name):
    # the benchmark's launch at full size (same inputs, dO and scale as bench.py --pass
    # bwd); every gradient of three whole heads (first, one inside, last) against the
    # oracle, and all of dQ, dK, dV finite
    import torch

    import exact_attention_90_amd as fa

    w = WORKLOADS[name] if name in WORKLOADS else HEADDIM_WORKLOADS[name]
    scale = float(np.float32(w.scale))
    say(f"bwd {name}: generating {w.short()}")
    x = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    g_np = make_dout(w.B, w.H, w.N, w.d, w.seed + 5000)
    xd = to_device(x, w.dtype)
    o, lse = fa.fwd(xd["q"], xd["k"], xd["v"], scale)
    g = torch.from_numpy(g_np).to("cuda")
    say(f"bwd {name}: fused backward")
    grads = fa.bwd(xd["q"], xd["k"], xd["v"], o, lse, g, scale)
    torch.cuda.synchronize()
    heads = [0, (w.B * w.H) // 2 + 1, w.B * w.H - 1]
    idx = torch.tensor(heads, device="cuda")
    sel = [t.reshape(w.B * w.H, w.N, w.d).index_select(0, idx).cpu().numpy() for t in grads]
    for t in grads:
        assert bool(torch.isfinite(t).all())
    say(f"bwd {name}: oracle on heads {heads}")
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], g_np, w.dtype, scale, heads=heads)
    assert_grads(sel, ref, w.dtype, f"{name} heads {heads}")
