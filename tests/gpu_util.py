"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run the
library through the Python binding, compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
from synth.inputs import make_qkv, to_torch

# Tolerances of the parity bar (fp32 inputs / 16-bit inputs).  LSE is compared by
# max |dLSE| / max(|LSE_ref|, 1) per element.
TOL_MAX_ABS = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
TOL_COSINE = 0.999
TOL_LSE_REL = 1e-4


def say(msg: str):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x, dtype):
    import torch

    return {n: to_torch(x[n], dtype).to("cuda") for n in ("q", "k", "v")}


def run(path: str, xd, scale):
    import torch

    import exact_attention_90_amd as fa

    f = fa.fwd if path == "fused" else fa.naive_fwd
    o, lse = f(xd["q"], xd["k"], xd["v"], scale)
    torch.cuda.synchronize()
    return o, lse


def metrics(o, lse, o_ref, lse_ref):
    o = np.asarray(o, np.float64).reshape(-1)
    r = np.asarray(o_ref, np.float64).reshape(-1)
    max_abs = float(np.abs(o - r).max()) if o.size else 0.0
    denom = float(np.linalg.norm(o) * np.linalg.norm(r))
    cosine = float(o @ r / denom) if denom > 0 else 1.0
    lse = np.asarray(lse, np.float64).reshape(-1)
    lr = np.asarray(lse_ref, np.float64).reshape(-1)
    lse_rel = float((np.abs(lse - lr) / np.maximum(np.abs(lr), 1.0)).max()) if lse.size else 0.0
    finite = bool(np.isfinite(o).all() and np.isfinite(lse).all())
    return dict(max_abs=max_abs, cosine=cosine, lse_rel=lse_rel, finite=finite)


def assert_parity(m, dtype, max_abs=None, where="", lse_rel=TOL_LSE_REL):
    tol = TOL_MAX_ABS[dtype] if max_abs is None else max_abs
    assert m["finite"], f"{where}: non-finite output"
    assert m["max_abs"] <= tol, f"{where}: max_abs {m['max_abs']:.3e} > {tol:g} ({m})"
    if dtype != "f32":
        assert m["cosine"] >= TOL_COSINE, f"{where}: cosine {m['cosine']:.6f} ({m})"
    assert m["lse_rel"] <= lse_rel, f"{where}: lse_rel {m['lse_rel']:.3e} ({m})"


def sample_rows(B, H, N, per_head=24, heads=12, seed=0):
    """Row indices (b*H + h)*N + i: tile edges, the ragged tail and random rows of a
    spread of heads (first, last and random ones)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nh = B * H
    hs = sorted(set([0, nh - 1] + list(rng.integers(0, nh, size=max(0, heads - 2)))))
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1]
    rows = []
    for hd in hs:
        ii = set(i for i in fixed if 0 <= i < N)
        ii.update(int(i) for i in rng.integers(0, N, size=per_head - len(ii)))
        rows.extend(hd * N + i for i in sorted(ii))
    return np.array(sorted(set(rows)), np.int64)


def spread_rows(B, H, N, count, seed=0):
    """At least `count` distinct row indices (b*H + h)*N + i over every head: each head's
    rows 0, 1, N-2, N-1 and its 64-row tile edges, the rest drawn at random, sorted."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nh = B * H
    per = max(4, -(-count // nh))
    rows = []
    for hd in range(nh):
        ii = {0, 1, N - 2, N - 1} | set(range(0, N, 64)) | set(range(63, N, 64))
        ii = {i for i in ii if 0 <= i < N}
        while len(ii) < min(per, N):
            ii.update(int(i) for i in rng.integers(0, N, size=min(per, N) - len(ii)))
        rows.extend(hd * N + i for i in sorted(ii))
    return np.array(sorted(set(rows)), np.int64)


def full_case(B, H, N, d, dtype, seed, mult=1.0, scale=None, path="fused", x=None):
    """Run a whole small problem on the GPU and the oracle; return metrics."""
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    scale32 = float(np.float32(scale))
    if x is None:
        x = make_qkv(B, H, N, d, dtype, seed, mult)
    say(f"{path} B={B} H={H} N={N} d={d} {dtype} seed={seed} mult={mult}")
    o, lse = run(path, to_device(x, dtype), scale32)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], dtype, scale32)
    return metrics(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref), x, (o, lse)
