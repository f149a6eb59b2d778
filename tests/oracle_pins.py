"""Pins that tie the CPU oracle to facts fixed outside itself.

Each pin returns None on success and raises AssertionError otherwise.  They are
collected by tests/test_oracle.py and re-run against deliberately broken builds
of the oracle by the mutation test (every broken build must fail at least one).

Sources of truth used here, none of which call into the oracle's code:
  * brute force on tiny inputs: exact sums (math.fsum) and the plain softmax
    definition without max subtraction, and mpmath at 50 digits;
  * library routines: scipy.special.softmax / logsumexp on a numpy score matrix;
  * closed forms: Q = 0 gives the column mean of V and LSE = ln N, constant V
    gives that constant, two keys give a logistic weighting, identical keys give
    the plain mean;
  * invariants: rows of P sum to one, joint K/V row permutation, key shift;
  * the online-softmax recurrences agree with the full-row max and sum-exp after
    every block, and reach the three-step O and LSE;
  * backward: torch autograd in float64 on the CPU, central finite differences of the
    forward oracle, closed forms (dO = 0; equal V rows give dQ = dK = 0; one key
    gives dV = dO) and invariants (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, key
    shift leaves every gradient unchanged).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from synth.inputs import make_qkv, quantize, to_float32


def _f64(bits, dtype):
    return to_float32(bits, dtype).astype(np.float64)


# ---------------------------------------------------------------- brute force
def _brute_fsum(qf, kf, vf, scale):
    """Exact-sum brute force of one head: softmax by its definition exp(s)/sum exp(s)."""
    N, d = qf.shape
    O = np.empty((N, d))
    L = np.empty(N)
    for i in range(N):
        s = [scale * math.fsum(float(qf[i, t]) * float(kf[j, t]) for t in range(d))
             for j in range(N)]
        e = [math.exp(x) for x in s]
        z = math.fsum(e)
        for t in range(d):
            O[i, t] = math.fsum(e[j] * float(vf[j, t]) for j in range(N)) / z
        L[i] = math.log(z)
    return O, L


def _brute_mp(qf, kf, vf, scale, dps=50):
    import mpmath

    with mpmath.workdps(dps):
        N, d = qf.shape
        O = np.empty((N, d))
        L = np.empty(N)
        sc = mpmath.mpf(scale)
        for i in range(N):
            s = [sc * mpmath.fsum(mpmath.mpf(float(qf[i, t])) * mpmath.mpf(float(kf[j, t]))
                                  for t in range(d)) for j in range(N)]
            e = [mpmath.exp(x) for x in s]
            z = mpmath.fsum(e)
            for t in range(d):
                O[i, t] = float(mpmath.fsum(e[j] * mpmath.mpf(float(vf[j, t]))
                                            for j in range(N)) / z)
            L[i] = float(mpmath.log(z))
    return O, L


def pin_brute_force(cases=None):
    """Oracle O/LSE equal brute force at N <= 64 (fsum) and on tiny cases (mpmath)."""
    if cases is None:
        cases = [("f32", 1, 2, 64, 16, 0.25, "fsum"), ("f16", 1, 1, 48, 64, 0.125, "fsum"),
                 ("bf16", 2, 1, 33, 8, 0.35, "fsum"), ("f16", 1, 1, 7, 5, 0.6, "mp"),
                 ("bf16", 1, 1, 5, 3, 1.7, "mp"), ("f32", 1, 1, 1, 4, 0.5, "mp")]
    for dtype, B, H, N, d, scale, how in cases:
        x = make_qkv(B, H, N, d, dtype, seed=100 + N + d, mult=1.5)
        o, lse = oracle.attention(x["q"], x["k"], x["v"], dtype, scale)
        qf, kf, vf = (_f64(x[n], dtype) for n in "qkv")
        for b in range(B):
            for h in range(H):
                f = _brute_fsum if how == "fsum" else _brute_mp
                Ob, Lb = f(qf[b, h], kf[b, h], vf[b, h], scale)
                vmax = max(1.0, np.abs(vf[b, h]).max())
                err_o = np.abs(o[b, h] - Ob).max() / vmax
                err_l = np.abs(lse[b, h] - Lb).max() / max(1.0, np.abs(Lb).max())
                assert err_o <= 1e-12, f"brute force O mismatch {err_o:.3e} ({dtype},{N},{d})"
                assert err_l <= 1e-12, f"brute force LSE mismatch {err_l:.3e} ({dtype},{N},{d})"


# ------------------------------------------------------ storage-format widening
def pin_storage_widening_every_pattern():
    """Every finite binary16 and bfloat16 bit pattern (subnormals and signed zeros
    included) reaches the arithmetic as the value a library gives it.  With Q = 0 every
    score is 0, so each query row's O is the plain mean of the V rows; with the same
    pattern in every V row that mean is the pattern's value exactly.  The reference
    values come from numpy's float16 and torch's bfloat16 conversions to float64."""
    import torch

    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        finite = (allbits & 0x7F80) != 0x7F80 if dtype == "bf16" else (allbits & 0x7C00) != 0x7C00
        bits = allbits[finite]
        if dtype == "f16":
            ref = bits.view(np.float16).astype(np.float64)
        else:
            ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(
                torch.float64).numpy()
        d = 512
        pad = (-len(bits)) % d
        bits = np.concatenate([bits, np.zeros(pad, np.uint16)])
        ref = np.concatenate([ref, np.zeros(pad)])
        H = len(bits) // d
        N = 2  # two identical key rows: O = (v + v) / 2 = v
        v = np.ascontiguousarray(np.broadcast_to(bits.reshape(1, H, 1, d), (1, H, N, d)))
        q = np.zeros((1, H, N, d), np.uint16)
        k = np.ascontiguousarray(v[:, :, ::-1])  # any keys: Q = 0 makes every score 0
        o, lse = oracle.attention(q, k, v, dtype, 0.5)
        want = np.broadcast_to(ref.reshape(1, H, 1, d), o.shape)
        bad = np.flatnonzero(o.reshape(-1) != want.reshape(-1))
        assert bad.size == 0, (f"{dtype}: {bad.size} patterns widened wrongly, e.g. element "
                               f"{bad[0]}: {o.reshape(-1)[bad[0]]!r} vs {want.reshape(-1)[bad[0]]!r}")
        assert np.all(lse == math.log(N)), f"{dtype}: LSE of all-zero scores is not ln N"
    # subnormal binary16 values enter the scores exactly too: q = 2^-24 (the smallest
    # subnormal) times k = 2^15 gives 2^-9 per column, 2^-7 over four columns
    q = np.full((1, 1, 1, 4), 0x0001, np.uint16)
    k = np.full((1, 1, 1, 4), np.float16(2.0**15).view(np.uint16), np.uint16)
    v = np.full((1, 1, 1, 4), np.float16(1.0).view(np.uint16), np.uint16)
    s, _, _, _ = oracle.head_steps(q, k, v, "f16", 1.0)
    assert s[0, 0] == 2.0**-7, f"subnormal query score {s[0, 0]!r} != 2^-7"


# ------------------------------------------------------------ the rows= entry
def pin_selected_rows_match_brute_force():
    """oracle.attention(rows=...) on unsorted rows spanning several heads (duplicates,
    first and last rows of heads) returns, in the order asked, each row's brute-force
    result."""
    B, H, N, d = 2, 2, 21, 8
    rows = np.array([83, 0, 20, 21, 22, 41, 42, 83, 5, 62, 63, 20, 0, 70, 41], np.int64)
    for dtype in ("f32", "f16", "bf16"):
        x = make_qkv(B, H, N, d, dtype, seed=7, mult=1.3)
        qf, kf, vf = (_f64(x[n], dtype) for n in "qkv")
        scale = 0.3
        o, lse = oracle.attention(x["q"], x["k"], x["v"], dtype, scale, rows=rows)
        assert o.shape == (len(rows), d) and lse.shape == (len(rows),)
        brute = {}
        for r_i, g in enumerate(rows):
            hd, i = divmod(int(g), N)
            if hd not in brute:
                b, h = divmod(hd, H)
                brute[hd] = _brute_fsum(qf[b, h], kf[b, h], vf[b, h], scale)
            Ob, Lb = brute[hd]
            err_o = np.abs(o[r_i] - Ob[i]).max() / max(1.0, np.abs(vf).max())
            err_l = abs(lse[r_i] - Lb[i]) / max(1.0, abs(Lb[i]))
            assert err_o <= 1e-12 and err_l <= 1e-12, (
                f"{dtype} row {g} (position {r_i}): O err {err_o:.3e}, LSE err {err_l:.3e}")


# ----------------------------------------------------------- library routines
def pin_scipy_softmax_logsumexp():
    """S equals scale*QK^T (numpy matmul), P equals scipy softmax(S), LSE equals logsumexp(S)."""
    from scipy.special import logsumexp, softmax

    for dtype, N, d, scale in (("f16", 96, 64, 0.125), ("bf16", 40, 128, 0.0884), ("f32", 50, 24, 0.3)):
        x = make_qkv(1, 1, N, d, dtype, seed=7 * N + d, mult=2.0)
        s, p, o, lse = oracle.head_steps(x["q"], x["k"], x["v"], dtype, scale)
        qf, kf, vf = (_f64(x[n], dtype)[0, 0] for n in "qkv")
        s_ref = scale * (qf @ kf.T)
        assert np.abs(s - s_ref).max() <= 1e-12 * max(1.0, np.abs(s_ref).max()), "S != scale QK^T"
        assert np.abs(p - softmax(s_ref, axis=1)).max() <= 1e-12, "P != scipy softmax"
        assert np.abs(lse - logsumexp(s_ref, axis=1)).max() <= 1e-12 * np.abs(lse).max(), \
            "LSE != scipy logsumexp"
        assert np.abs(o - softmax(s_ref, axis=1) @ vf).max() <= 1e-12 * np.abs(vf).max(), \
            "O != softmax(S) V"
        # the sampled-row entry point agrees with the head entry point
        o2, l2 = oracle.attention(x["q"], x["k"], x["v"], dtype, scale)
        assert np.abs(o2[0, 0] - o).max() <= 1e-13 and np.abs(l2[0, 0] - lse).max() <= 1e-13


# ----------------------------------------------------------------- closed forms
def pin_rows_sum_to_one():
    x = make_qkv(1, 1, 77, 32, "bf16", seed=5, mult=3.0)
    s, p, o, lse = oracle.head_steps(x["q"], x["k"], x["v"], "bf16", 0.2)
    assert np.all(p >= 0.0)
    assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-13 * 77, "rows of P do not sum to 1"


def pin_zero_query():
    """Q = 0: every score is 0, so O = column mean of V (over the N keys) and LSE = ln N."""
    for dtype in ("f32", "f16", "bf16"):
        B, H, N, d = 2, 3, 37, 16
        x = make_qkv(B, H, N, d, dtype, seed=3)
        zero = quantize(np.zeros((B, H, N, d), np.float32), dtype)
        o, lse = oracle.attention(zero, x["k"], x["v"], dtype, 0.25)
        vf = _f64(x["v"], dtype)
        mean = vf.mean(axis=2, keepdims=True)
        assert np.abs(o - mean).max() <= 1e-12, "Q=0 does not give the column mean of V"
        assert np.abs(lse - math.log(N)).max() <= 1e-12, "Q=0 does not give LSE = ln N"
        # K = 0 is the same closed form
        o, lse = oracle.attention(x["q"], zero, x["v"], dtype, 0.25)
        assert np.abs(o - mean).max() <= 1e-12 and np.abs(lse - math.log(N)).max() <= 1e-12


def pin_constant_v():
    for dtype, c in (("f32", -2.75), ("f16", 3.5), ("bf16", 0.15625)):
        B, H, N, d = 1, 2, 29, 8
        x = make_qkv(B, H, N, d, dtype, seed=9, mult=4.0)
        vc = quantize(np.full((B, H, N, d), c, np.float32), dtype)
        o, _ = oracle.attention(x["q"], x["k"], vc, dtype, 0.5)
        assert np.abs(o - c).max() <= 1e-12 * abs(c) * 4, "constant V not returned"


def pin_two_keys():
    """N = 2, d = 1: q = 1, keys (0, a) give weights (1, e^{sa}) / (1 + e^{sa}).
    Query 2 has q = -1, so its weights are (1, e^{-sa}) / (1 + e^{-sa})."""
    a, v0, v1, scale = 1.5, 2.0, -3.0, 0.75
    q = np.array([1.0, -1.0], np.float32).reshape(1, 1, 2, 1)
    k = np.array([0.0, a], np.float32).reshape(1, 1, 2, 1)
    v = np.array([v0, v1], np.float32).reshape(1, 1, 2, 1)
    o, lse = oracle.attention(q, k, v, "f32", scale)
    for i, sgn in enumerate((1.0, -1.0)):
        w1 = 1.0 / (1.0 + math.exp(-sgn * scale * a))  # logistic weight of key 1
        assert abs(o[0, 0, i, 0] - ((1 - w1) * v0 + w1 * v1)) <= 1e-15 * 4
        assert abs(lse[0, 0, i] - math.log(1.0 + math.exp(sgn * scale * a))) <= 1e-15 * 4


def pin_identical_keys_large_logits():
    """All keys equal and logits huge (s ~ 2.6e3): the max subtraction keeps it finite;
    O is the plain mean of V and LSE = s + ln N."""
    N, d = 24, 64
    q = np.full((1, 1, N, d), 6.5, np.float32)
    k = np.full((1, 1, N, d), 6.25, np.float32)
    v = make_qkv(1, 1, N, d, "f32", seed=1)["v"]
    o, lse = oracle.attention(q, k, v, "f32", 1.0)
    s = 6.5 * 6.25 * d
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.abs(o[0, 0] - v[0, 0].astype(np.float64).mean(axis=0)).max() <= 1e-12
    assert np.abs(lse[0, 0] - (s + math.log(N))).max() <= 1e-12 * s


def pin_large_spread_logits():
    """Scores 1000, 0, -1000 (d = 1, q = 1): without subtracting the row max, exp would
    overflow.  The first key takes all the weight in double precision, so O = v_0
    exactly and LSE = 1000 (e^-1000 is below double's range)."""
    q = np.ones((1, 1, 3, 1), np.float32)
    k = np.array([1000.0, 0.0, -1000.0], np.float32).reshape(1, 1, 3, 1)
    v = np.array([1.25, -7.0, 3.0], np.float32).reshape(1, 1, 3, 1)
    o, lse = oracle.attention(q, k, v, "f32", 1.0)
    assert np.all(o[0, 0, :, 0] == 1.25), f"large-spread O wrong: {o.ravel()}"
    assert np.all(lse[0, 0] == 1000.0), f"large-spread LSE wrong: {lse.ravel()}"


# ----------------------------------------------------------------- invariants
def pin_permutation_invariance():
    x = make_qkv(1, 2, 45, 16, "f16", seed=21)
    o, lse = oracle.attention(x["q"], x["k"], x["v"], "f16", 0.3)
    perm = np.random.Generator(np.random.PCG64(4)).permutation(45)
    o2, lse2 = oracle.attention(x["q"], x["k"][:, :, perm], x["v"][:, :, perm], "f16", 0.3)
    assert np.abs(o - o2).max() <= 1e-13 and np.abs(lse - lse2).max() <= 1e-13
    # a K-only permutation must change the result (guards against ignoring the pairing)
    o3, _ = oracle.attention(x["q"], x["k"][:, :, perm], x["v"], "f16", 0.3)
    assert np.abs(o - o3).max() > 1e-3


def pin_key_shift():
    """K += 1 u^T leaves O unchanged and moves LSE_i by scale * <q_i, u>.
    Integer-valued inputs keep every value exact in float32."""
    rng = np.random.Generator(np.random.PCG64(8))
    N, d, scale = 31, 12, 0.375
    q = rng.integers(-3, 4, (1, 1, N, d)).astype(np.float32)
    k = rng.integers(-3, 4, (1, 1, N, d)).astype(np.float32)
    v = rng.integers(-5, 6, (1, 1, N, d)).astype(np.float32)
    u = rng.integers(-2, 3, d).astype(np.float32)
    o, lse = oracle.attention(q, k, v, "f32", scale)
    o2, lse2 = oracle.attention(q, k + u, v, "f32", scale)
    shift = scale * (q[0, 0].astype(np.float64) @ u.astype(np.float64))
    assert np.abs(o - o2).max() <= 1e-12
    assert np.abs((lse2 - lse)[0, 0] - shift).max() <= 1e-12 * max(1.0, np.abs(lse).max())


# ------------------------------------------------------------ online softmax
def pin_online_equals_three_step():
    """Blockwise recurrences: after block j, m is the max of the scores seen so far
    (exactly) and l is their sum of exp(s - m); the end result is the three-step O and LSE."""
    for dtype, N, d in (("f16", 64, 16), ("bf16", 50, 8), ("f32", 17, 4)):
        x = make_qkv(1, 1, N, d, dtype, seed=N, mult=2.5)
        scale = 1.0 / math.sqrt(d)
        s, p, o3, l3 = oracle.head_steps(x["q"], x["k"], x["v"], dtype, scale)
        for block in (1, 3, 16, 64, N):
            o, lse, mt, lt = oracle.online_head(x["q"], x["k"], x["v"], dtype, scale, block)
            nb = mt.shape[1]
            for jb in range(nb):
                hi = min(N, (jb + 1) * block)
                pref = s[:, :hi]
                mref = pref.max(axis=1)
                assert np.array_equal(mt[:, jb], mref), f"online m != prefix max (block {block})"
                lref = np.exp(pref - mref[:, None]).sum(axis=1)
                assert np.abs(lt[:, jb] - lref).max() <= 1e-12 * lref.max(), \
                    f"online l != prefix sum-exp (block {block})"
            assert np.abs(o - o3).max() <= 1e-12 * max(1.0, np.abs(o3).max()), \
                f"online O != three-step O (block {block})"
            assert np.abs(lse - l3).max() <= 1e-12 * np.abs(l3).max()


# ---------------------------------------------------------------- backward
# The backward oracle is tied to torch's autograd (float64, CPU: a library routine that
# shares nothing with the oracle), to central finite differences of the forward oracle
# (which the pins above tie down), and to closed forms and invariants of the gradient.
def _torch_grads(q, k, v, dout, dtype, scale):
    import torch

    qf, kf, vf = (torch.tensor(_f64(a, dtype), requires_grad=True) for a in (q, k, v))
    p = torch.softmax(scale * (qf @ kf.transpose(-1, -2)), dim=-1)
    o = p @ vf
    o.backward(torch.tensor(dout.astype(np.float64)))
    return qf.grad.numpy(), kf.grad.numpy(), vf.grad.numpy()


def _rel_err(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def pin_bwd_torch_autograd():
    from synth.inputs import make_dout

    for (B, H, N, d, dtype, mult, seed) in [(1, 2, 7, 5, "f32", 1.0, 51), (2, 1, 33, 16, "bf16", 1.0, 52),
                                            (1, 1, 64, 64, "f16", 2.0, 53), (1, 2, 20, 8, "f32", 4.0, 54)]:
        x = make_qkv(B, H, N, d, dtype, seed, mult)
        g = make_dout(B, H, N, d, seed + 1000)
        scale = 1.0 / math.sqrt(d)
        ours = oracle.attention_bwd(x["q"], x["k"], x["v"], g, dtype, scale)
        ref = _torch_grads(x["q"], x["k"], x["v"], g, dtype, scale)
        for name, a, b in zip(("dq", "dk", "dv"), ours, ref):
            e = _rel_err(a, b)
            assert e < 1e-11, f"{name} vs torch autograd ({B},{H},{N},{d},{dtype}): {e:.3e}"
    # a subset of heads returns exactly those heads
    x = make_qkv(2, 3, 9, 4, "f32", 55)
    g = make_dout(2, 3, 9, 4, 1055)
    full = oracle.attention_bwd(x["q"], x["k"], x["v"], g, "f32", 0.5)
    part = oracle.attention_bwd(x["q"], x["k"], x["v"], g, "f32", 0.5, heads=[1, 4])
    for a, b in zip(full, part):
        assert np.array_equal(a.reshape(6, 9, 4)[[1, 4]], b)


def pin_bwd_finite_differences():
    """Central differences of L = sum(O * dO) through the forward oracle, on float32
    inputs (the step actually taken is the float32-rounded one)."""
    from synth.inputs import make_dout

    B, H, N, d = 1, 2, 5, 3
    x = make_qkv(B, H, N, d, "f32", 61)
    g = make_dout(B, H, N, d, 1061)
    scale = 0.7
    grads = dict(zip("qkv", oracle.attention_bwd(x["q"], x["k"], x["v"], g, "f32", scale)))

    def loss(xx):
        o, _ = oracle.attention(xx["q"], xx["k"], xx["v"], "f32", scale)
        return float(np.sum(o * g.astype(np.float64)))

    for name in "qkv":
        fd = np.empty((B, H, N, d))
        for idx in np.ndindex(B, H, N, d):
            x0 = float(x[name][idx])
            vals = []
            for sgn in (+1, -1):
                xx = {n: x[n].copy() for n in "qkv"}
                xx[name][idx] = np.float32(x0 + sgn * 1e-3)
                vals.append((loss(xx), float(xx[name][idx])))
            (lp, xp), (lm, xm) = vals
            fd[idx] = (lp - lm) / (xp - xm)
        e = np.abs(fd - grads[name]).max() / np.abs(grads[name]).max()
        assert e < 1e-5, f"d{name} vs finite differences: {e:.3e}"


def pin_bwd_closed_forms():
    from synth.inputs import make_dout

    B, H, N, d = 1, 2, 24, 8
    x = make_qkv(B, H, N, d, "f32", 71, mult=2.0)
    scale = 1.0 / math.sqrt(d)
    # dO = 0: every gradient is zero
    z = np.zeros((B, H, N, d), np.float32)
    for a in oracle.attention_bwd(x["q"], x["k"], x["v"], z, "f32", scale):
        assert not np.any(a)
    g = make_dout(B, H, N, d, 1071)
    # every V row the same: O is that row whatever P is, so dQ = dK = 0, and
    # sum_j dV_j = sum_i dO_i (the rows of P sum to one)
    xc = dict(x)
    xc["v"] = np.ascontiguousarray(np.broadcast_to(x["v"][:, :, :1], x["v"].shape))
    dq, dk, dv = oracle.attention_bwd(xc["q"], xc["k"], xc["v"], g, "f32", scale)
    tiny = 1e-12 * np.abs(g).max() * np.abs(_f64(x["k"], "f32")).max()
    assert np.abs(dq).max() < tiny and np.abs(dk).max() < tiny, (np.abs(dq).max(), np.abs(dk).max())
    assert np.allclose(dv.sum(axis=2), g.astype(np.float64).sum(axis=2), rtol=0, atol=1e-12)
    # one key: P = 1, so dV = the sum of dO over the (single) query and dQ = dK = 0
    x1 = make_qkv(1, 1, 1, 6, "f32", 72)
    g1 = make_dout(1, 1, 1, 6, 1072)
    dq, dk, dv = oracle.attention_bwd(x1["q"], x1["k"], x1["v"], g1, "f32", 0.3)
    assert not np.any(dq) and not np.any(dk)
    assert np.array_equal(dv, g1.astype(np.float64))


def pin_bwd_invariants():
    from synth.inputs import make_dout

    B, H, N, d = 2, 1, 37, 12
    x = make_qkv(B, H, N, d, "f32", 81, mult=1.5)
    g = make_dout(B, H, N, d, 1081)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_bwd(x["q"], x["k"], x["v"], g, "f32", scale)
    mag = np.abs(dk).max()
    # each row of dS sums to zero, so sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12 * N * mag
    # the rows of P sum to one: sum_j dV_j = sum_i dO_i
    assert np.allclose(dv.sum(axis=2), g.astype(np.float64).sum(axis=2), rtol=0, atol=1e-11)
    # key shift K + 1 u^T moves every score of a row by the same amount: P, dS and all
    # three gradients are unchanged (dQ because the rows of dS sum to zero).  Keys and
    # shift lie on a 2^-8 grid, so the shifted keys are exact in float32.
    grid = lambda a: (np.round(np.asarray(a, np.float64) * 256) / 256).astype(np.float32)
    k0 = grid(x["k"])
    u = grid(np.random.Generator(np.random.PCG64(82)).standard_normal(d))
    k1 = (k0 + u).astype(np.float32)
    assert np.array_equal(k1.astype(np.float64), k0.astype(np.float64) + u.astype(np.float64))
    base = oracle.attention_bwd(x["q"], k0, x["v"], g, "f32", scale)
    moved = oracle.attention_bwd(x["q"], k1, x["v"], g, "f32", scale)
    for name, a, b in zip(("dq", "dk", "dv"), moved, base):
        assert _rel_err(a, b) < 1e-10, f"key shift changed {name}: {_rel_err(a, b):.3e}"


ALL_PINS = [
    pin_brute_force,
    pin_storage_widening_every_pattern,
    pin_selected_rows_match_brute_force,
    pin_scipy_softmax_logsumexp,
    pin_rows_sum_to_one,
    pin_zero_query,
    pin_constant_v,
    pin_two_keys,
    pin_identical_keys_large_logits,
    pin_large_spread_logits,
    pin_permutation_invariance,
    pin_key_shift,
    pin_online_equals_three_step,
    pin_bwd_torch_autograd,
    pin_bwd_finite_differences,
    pin_bwd_closed_forms,
    pin_bwd_invariants,
]
