"""Parity of the fused HIP kernel (fa_fwd) with the CPU fp64 oracle.

Bar: max |O - O_ref| <= 1e-5 for fp32 inputs and <= 1e-2 (cosine >= 0.999) for
fp16/bf16 inputs; LSE within 1e-4 relative.  Small problems are compared element
by element in full; the five named workloads run at full size and are compared on
sampled rows computed one by one by the oracle.
"""
import math

import numpy as np
import pytest

import oracle
from synth.configs import PAGE_WORKLOADS, WORKLOADS
from synth.inputs import make_qkv, quantize, to_float32
from tests.gpu_util import (assert_parity, full_case, metrics, run, say, spread_rows,
                            to_device)

pytestmark = pytest.mark.gpu


# ---- small problems, every element ------------------------------------------------
@pytest.mark.parametrize("B,H,N,d,dtype", [
    (2, 3, 333, 128, "f16"), (2, 3, 333, 128, "bf16"), (1, 2, 333, 64, "f16"),
    (1, 2, 333, 64, "bf16"), (2, 2, 200, 64, "f32"), (1, 2, 300, 128, "f32"),
    (1, 2, 512, 128, "bf16"), (1, 2, 512, 64, "f16"), (1, 1, 1000, 128, "f16"),
])
def test_small_full(B, H, N, d, dtype):
    m, _, _ = full_case(B, H, N, d, dtype, seed=N + d)
    assert_parity(m, dtype, where=f"{B}x{H}x{N}x{d} {dtype}")


def test_c1_tiny_fp32_full():
    w = WORKLOADS["c1"]
    m, _, _ = full_case(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    assert_parity(m, w.dtype, where="c1")


@pytest.mark.parametrize("name", sorted(PAGE_WORKLOADS))
def test_page_workloads(name):
    w = PAGE_WORKLOADS[name]
    m, _, _ = full_case(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    assert_parity(m, w.dtype, where=name)


@pytest.mark.parametrize("N,d", [(64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_single_key_tile(N, d, dtype):
    # N equal to one key tile: the loop runs once (the tutorial's N_CTX = BLOCK_N check)
    m, _, _ = full_case(1, 2, N, d, dtype, seed=5)
    assert_parity(m, dtype, where=f"single tile N={N} d={d}")


@pytest.mark.parametrize("N", [1, 2, 3, 31, 33, 127, 129])
@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 64), ("f32", 64)])
def test_tiny_and_ragged(N, dtype, d):
    m, x, (o, lse) = full_case(1, 3, N, d, dtype, seed=100 + N)
    assert_parity(m, dtype, where=f"N={N}")
    if N == 1:
        # one key: O is that key's value row.  16-bit P rounds 2^(fma residue) to exactly
        # 1, so O = v (bf16 values below binary16's normal range round when widened for
        # the P V product); fp32 P keeps the residue of s*c, a relative 2^-24, so O = v
        # within an ulp or two.
        v = to_float32(x["v"], dtype).astype(np.float64)
        err = np.abs(o.cpu().numpy().astype(np.float64) - v).max()
        tol = {"f16": 0.0, "bf16": 2.0**-25, "f32": 2.0**-22 * np.abs(v).max()}[dtype]
        assert err <= tol


# key-tile counts 2, 3, 5, 8 and 10 (ragged and exact last tiles) and partial query
# tiles of both workgroup sizes: every length of the software-pipelined loop, with the
# masked iteration alone (2 tiles) and after odd and even numbers of steady iterations
@pytest.mark.parametrize("N", [65, 191, 257, 449, 640])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 64)])
def test_pipeline_lengths(N, dtype, d):
    m, _, _ = full_case(1, 2, N, d, dtype, seed=300 + N)
    assert_parity(m, dtype, where=f"N={N} d={d} {dtype}")


@pytest.mark.parametrize("dtype,mult,d", [("bf16", 3.0, 128), ("f16", 8.0, 128), ("bf16", 12.0, 128),
                                          ("f16", 8.0, 64), ("bf16", 12.0, 64)])
def test_large_logits(dtype, mult, d):
    # logit standard deviation ~ mult^2: needs the running-max subtraction and rescale
    # (at d = 64 with the row max of each wave's two query blocks taken in different steps)
    m, _, _ = full_case(1, 2, 2000, d, dtype, seed=77, mult=mult)
    assert_parity(m, dtype, where=f"x{mult} d={d}")


@pytest.mark.parametrize("scale", [1e-6, 50.0])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_extreme_scales(dtype, d, scale):
    # scale 1e-6: every logit ~0, P ~1 everywhere (O is the column mean, LSE ~ ln N, the
    # row sum over every key); scale 50: logit spread ~50 sqrt(d), one key per row
    # dominates and the running max jumps by far more than the lagging reference's reach
    m, x, _ = full_case(1, 2, 333, d, dtype, seed=900 + d, scale=scale)
    tol = None
    if dtype == "f32" and scale > 1.0:
        # the 1e-5 bar assumes moderate logits.  Here each logit is an fp32 dot product
        # with |ds_j| <= scale (d + 1) u sum_k |q_k k_jk| (u = 2^-24), ~1e-2 at scale 50,
        # and to first order |dO| <= sum_j p_j (|ds_j| + sum_l p_l |ds_l|) |v_j - O|; that
        # bound (worst-case signs) is the tolerance, and the direction of O must still
        # agree to 1e-7 (a wrong rescale would not)
        q, k, v = (to_float32(x[n], dtype).astype(np.float64) for n in "qkv")
        sc = float(np.float32(scale))
        s_ = sc * np.einsum("bhid,bhjd->bhij", q, k)
        p_ = np.exp(s_ - s_.max(-1, keepdims=True))
        p_ /= p_.sum(-1, keepdims=True)
        o_ = np.einsum("bhij,bhjd->bhid", p_, v)
        dl = sc * (d + 1) * 2.0**-24 * np.einsum("bhid,bhjd->bhij", np.abs(q), np.abs(k))
        w_ = p_ * (dl + (p_ * dl).sum(-1, keepdims=True))
        tol = 1e-5
        for h in range(v.shape[1]):  # one head at a time: [N, N, d] per head
            diff = np.abs(v[0, h][None, :, :] - o_[0, h][:, None, :])
            tol = max(tol, float(np.einsum("ij,ijd->id", w_[0, h], diff).max()))
        assert m["cosine"] >= 1.0 - 1e-7, m
    assert_parity(m, dtype, max_abs=tol, where=f"scale={scale} d={d} {dtype}")


def test_empty_problem():
    import torch

    import exact_attention_90_amd as fa

    q = torch.empty((2, 3, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fwd(q, q, q)
    assert o.shape == (2, 3, 0, 128) and lse.shape == (2, 3, 0)


# ---- closed forms and invariants on the GPU ------------------------------------------
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_zero_query_gives_column_mean(dtype, d):
    B, H, N = 2, 2, 777
    x = make_qkv(B, H, N, d, dtype, seed=8)
    x["q"] = quantize(np.zeros((B, H, N, d), np.float32), dtype)
    say(f"Q=0 {dtype} d={d}")
    o, lse = run("fused", to_device(x, dtype), 1.0 / math.sqrt(d))
    mean = to_float32(x["v"], dtype).astype(np.float64).mean(axis=2, keepdims=True)
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert np.abs(o.cpu().numpy() - mean).max() <= tol
    assert np.abs(lse.cpu().numpy() - math.log(N)).max() <= 1e-4 * math.log(N)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_constant_v_returns_the_constant(dtype):
    B, H, N, d = 1, 2, 555, 128
    x = make_qkv(B, H, N, d, dtype, seed=9, mult=3.0)
    c = 1.75
    x["v"] = quantize(np.full((B, H, N, d), c, np.float32), dtype)
    say(f"V=const {dtype}")
    o, _ = run("fused", to_device(x, dtype), 1.0 / math.sqrt(d))
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert np.abs(o.cpu().numpy() - c).max() <= tol


def test_joint_kv_permutation_invariance():
    B, H, N, d, dtype = 1, 2, 640, 128, "bf16"
    x = make_qkv(B, H, N, d, dtype, seed=10)
    say("permutation")
    o1, l1 = run("fused", to_device(x, dtype), 1.0 / math.sqrt(d))
    perm = np.random.Generator(np.random.PCG64(3)).permutation(N)
    xp = dict(q=x["q"], k=np.ascontiguousarray(x["k"][:, :, perm]),
              v=np.ascontiguousarray(x["v"][:, :, perm]))
    o2, l2 = run("fused", to_device(xp, dtype), 1.0 / math.sqrt(d))
    assert np.abs(o1.cpu().numpy() - o2.cpu().numpy()).max() <= 2e-3
    assert np.abs(l1.cpu().numpy() - l2.cpu().numpy()).max() <= 1e-4 * 10


def test_bitwise_deterministic():
    import torch

    B, H, N, d, dtype = 2, 4, 1024, 128, "bf16"
    xd = to_device(make_qkv(B, H, N, d, dtype, seed=12), dtype)
    say("determinism")
    outs = [run("fused", xd, 1.0 / math.sqrt(d)) for _ in range(3)]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


# ---- the persistent form --------------------------------------------------------------
# 16-bit d = 128 and d = 256 problems with more query tiles (256 rows at d = 128, 128 at
# d = 256) than the device holds workgroups at once (256 on MI355X) run as one workgroup
# per slot taking its tiles in turn, the next tile's Q and first K/V tiles loaded while the
# current one finishes.  Below: 257 to 1200 tiles (one to five per workgroup), 2 to 16 key
# tiles, ragged last key and query tiles.
@pytest.mark.parametrize("B,H,N,d,dtype", [(1, 300, 65, 128, "bf16"), (1, 260, 128, 128, "f16"),
                                          (2, 150, 129, 128, "bf16"), (3, 100, 700, 128, "f16"),
                                          (1, 257, 256, 128, "bf16"), (2, 75, 1000, 128, "bf16"),
                                          (1, 300, 65, 256, "bf16"), (1, 257, 128, 256, "f16"),
                                          (2, 100, 700, 256, "bf16"), (3, 30, 1000, 256, "f16")])
def test_persistent_form_against_oracle(B, H, N, d, dtype):
    m, _, _ = full_case(B, H, N, d, dtype, seed=700 + N + d)
    assert_parity(m, dtype, where=f"persistent {B}x{H}x{N}x{d} {dtype}")


@pytest.mark.parametrize("H,N,d,chunk,dtype", [(600, 128, 128, 128, "f16"), (200, 700, 128, 64, "bf16"),
                                              (96, 2048, 128, 32, "bf16"), (300, 256, 256, 128, "bf16"),
                                              (48, 2048, 256, 16, "f16")])
def test_persistent_form_matches_one_tile_per_workgroup(H, N, d, chunk, dtype):
    # the whole batch (persistent form) against the same heads in calls of at most 256
    # query tiles (one tile per workgroup): the same arithmetic, so bitwise the same
    import torch

    xd = to_device(make_qkv(1, H, N, d, dtype, seed=900 + N + d), dtype)
    say(f"persistent vs per-tile H={H} N={N} d={d} {dtype}")
    o, lse = run("fused", xd, 1.0 / math.sqrt(d))
    for h0 in range(0, H, chunk):
        part = {n: t[:, h0:h0 + chunk] for n, t in xd.items()}
        op, lp = run("fused", part, 1.0 / math.sqrt(d))
        assert torch.equal(op, o[:, h0:h0 + chunk]) and torch.equal(lp, lse[:, h0:h0 + chunk]), h0


def test_persistent_forms_on_concurrent_streams():
    # two persistent launches (d = 128 and d = 256) and a per-tile one (d = 64) enqueued on
    # three streams at once, so that their workgroups share the compute units: each result
    # equals the same call made alone
    import torch

    import exact_attention_90_amd as fa

    cases = [(1, 300, 256, 128, "bf16"), (1, 300, 128, 256, "f16"), (2, 8, 1024, 64, "bf16")]
    xs = [to_device(make_qkv(B, H, N, d, dt, seed=60 + i), dt) for i, (B, H, N, d, dt) in enumerate(cases)]
    say("persistent forms on concurrent streams")
    alone = [run("fused", x, 1.0 / math.sqrt(c[3])) for x, c in zip(xs, cases)]
    streams = [torch.cuda.Stream() for _ in cases]
    outs = []
    for x, c, st in zip(xs, cases, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(fa.fwd(x["q"], x["k"], x["v"], 1.0 / math.sqrt(c[3])))
    torch.cuda.synchronize()
    for (o, lse), (o1, l1) in zip(outs, alone):
        assert torch.equal(o, o1) and torch.equal(lse, l1)


# ---- the named workloads at full size ----------------------------------------------
def _compare_rows(name, w, o, lse, x, rows):
    """Oracle on `rows` (None: every row) against the kernel's output."""
    import torch

    scale32 = float(np.float32(w.scale))
    say(f"{name}: oracle on {'every row' if rows is None else f'{len(rows)} rows'}")
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], w.dtype, scale32, rows=rows)
    if rows is None:
        o_s, l_s = o.cpu().numpy(), lse.cpu().numpy()
    else:
        idx = torch.from_numpy(rows).to(o.device)
        o_s = o.reshape(-1, w.d).index_select(0, idx).cpu().numpy()
        l_s = lse.reshape(-1).index_select(0, idx).cpu().numpy()
    m = metrics(o_s, l_s, o_ref, lse_ref)
    say(f"{name}: {m}")
    assert_parity(m, w.dtype, where=name)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


def _run_workload(name):
    w = WORKLOADS[name]
    say(f"{name}: generating {w.short()}")
    x = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult)
    say(f"{name}: fused kernel")
    o, lse = run("fused", to_device(x, w.dtype), float(np.float32(w.scale)))
    return w, x, o, lse


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_workload_every_row(name):
    # the whole output of the fp16 workloads against the oracle
    w, x, o, lse = _run_workload(name)
    _compare_rows(name, w, o, lse, x, None)


@pytest.mark.parametrize("name,nrows", [("c3", 120_000), ("c5", 100_000)])
def test_workload_many_rows(name, nrows):
    # at least 1e5 rows spread over every head: each head's first and last rows, the
    # edges of its query tiles and random rows
    w, x, o, lse = _run_workload(name)
    rows = spread_rows(w.B, w.H, w.N, nrows, seed=w.seed)
    assert len(rows) >= nrows
    _compare_rows(name, w, o, lse, x, rows)


def test_longest_accepted_head():
    # the largest head the boundary accepts for 16-bit inputs at d = 128: one head of Q, K
    # or V may take 2^31 - 2^17 bytes (the buffer-descriptor range less one tile), so
    # N = 2^23 - 512 (N + 1 is refused, a CPU test checks that) and O is ~4 GiB; 32766
    # query tiles of 131064 key tiles each.  Rows at both ends, at tile and workgroup
    # edges and at random against the oracle (~4 GFLOP of fp64 per row).
    import torch

    B, H, N, d, dtype = 1, 1, 2**23 - 512, 128, "bf16"
    scale32 = float(np.float32(1.0 / math.sqrt(d)))
    say(f"longest head: generating bf16 B1 H1 N{N} d{d}")
    x = make_qkv(B, H, N, d, dtype, seed=2323)
    say("longest head: fused kernel (~40 s)")
    o, lse = run("fused", to_device(x, dtype), scale32)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(23))
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, N // 2, N - 257, N - 256, N - 65, N - 64,
             N - 33, N - 32, N - 2, N - 1]
    rows = np.array(sorted(set(fixed) | set(int(i) for i in rng.integers(0, N, size=31))),
                    np.int64)
    say(f"longest head: oracle on {len(rows)} rows")
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], dtype, scale32, rows=rows)
    idx = torch.from_numpy(rows).to(o.device)
    m = metrics(o.reshape(-1, d).index_select(0, idx).cpu().numpy(),
                lse.reshape(-1).index_select(0, idx).cpu().numpy(), o_ref, lse_ref)
    say(f"longest head: {m}")
    assert_parity(m, dtype, where="N = 2^23 - 512")
    assert bool(torch.isfinite(lse).all())
