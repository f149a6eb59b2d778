"""The second validation layer: the kernel's online-softmax statistics after every 64-key
block (running max and running sum, CK/MI50 notes section 4.1, layer 2) against the CPU
oracle's blockwise recurrences (MUSA guide, online-softmax recurrences; oracle
online_head with block 64), read back through fa_fwd_stats.

Tolerances are bounds derived from the arithmetic, per row and block (u = 2^-24):
  * a score s_j = scale q.k_j is a float32 sum of d products (exact for 16-bit inputs,
    each rounded for fp32 inputs): |ds_j| <= scale (d + 1) u sum_k |q_k k_jk|.  The
    kernel's max is off by at most max_j |ds_j| over the block's prefix, plus the
    rounding of the product with log2(e) scale and of its conversion (2 u |m|).
  * the running sum is a float32 sum of n <= N terms exp2(fma(s_j, c, -ref)): each term's
    relative error is at most |d(s_j - m)| + ln2 u (|c s_j| + |ref|) + 2 u (the
    hardware exp2 is within one ulp), and the summation adds n u.
For 16-bit inputs at d >= 128 the kernel keeps a lagging reference (at most 8 base-2
units below the max), so there the running log-sum ref ln2 + ln l is compared with
m + ln l, and the reference is checked to lie within [m - 8 ln 2, m]."""
import math

import numpy as np
import pytest
import torch

import exact_attention_90_amd as fa
import oracle
from synth.inputs import make_qkv, to_float32
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

U = 2.0**-24
LN2 = math.log(2.0)
TAU = 8.0  # the lagging reference's reach (base-2 units)


@pytest.mark.parametrize("d,dtype", [(64, "f16"), (64, "bf16"), (128, "f16"), (128, "bf16"),
                                     (256, "f16"), (256, "bf16"), (64, "f32"), (128, "f32"),
                                     (256, "f32")])
def test_block_statistics_match_the_recurrences(d, dtype):
    B, H, N = 1, 2, 333  # six 64-key blocks, the last ragged (13 keys)
    x = make_qkv(B, H, N, d, dtype, seed=40 + d, mult=1.5)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    xd = to_device(x, dtype)
    say(f"fa_fwd_stats B={B} H={H} N={N} d={d} {dtype}")
    o, lse, st = fa.fwd_stats(xd["q"], xd["k"], xd["v"], scale)
    o0, lse0 = fa.fwd(xd["q"], xd["k"], xd["v"], scale)
    torch.cuda.synchronize()
    # the recording form computes exactly what fa_fwd computes
    assert torch.equal(o, o0) and torch.equal(lse, lse0)
    st = st.cpu().numpy().astype(np.float64)
    nb = (N + 63) // 64
    assert st.shape == (B, H, N, nb, 2)
    lagging = dtype != "f32" and d >= 128
    qf, kf = (to_float32(x[n], dtype).astype(np.float64) for n in "qk")
    for b in range(B):
        for h in range(H):
            _, _, mt, lt = oracle.online_head(x["q"], x["k"], x["v"], dtype, scale, 64,
                                              head=b * H + h)
            ref2, l_k = st[b, h, :, :, 0], st[b, h, :, :, 1]
            # per-score error bound and its running max over each block prefix
            ds = scale * (d + 1) * U * (np.abs(qf[b, h]) @ np.abs(kf[b, h]).T)  # [N, N]
            s_abs = scale * np.abs(qf[b, h] @ kf[b, h].T)
            ends = np.minimum(64 * np.arange(1, nb + 1), N)
            ds_pre = np.stack([ds[:, :e].max(axis=1) for e in ends], axis=1)
            sa_pre = np.stack([s_abs[:, :e].max(axis=1) for e in ends], axis=1)
            n_pre = ends[None, :].astype(np.float64)
            tol_m = ds_pre + 2 * U * np.abs(mt) + 1e-30
            # fma(s, c, -ref) in base-2 units: |c s| = |scaled s| log2(e)
            tol_l = (2 * ds_pre + LN2 * U * (sa_pre * math.log2(math.e) + np.abs(ref2))
                     + 2 * U + n_pre * U)
            m_k = ref2 * LN2
            if not lagging:
                err_m = np.abs(m_k - mt)
                worst = np.unravel_index(np.argmax(err_m / tol_m), err_m.shape)
                assert (err_m <= tol_m).all(), (
                    f"running max off by {err_m[worst]:.3e} > bound {tol_m[worst]:.3e} at {worst}")
                rel_l = np.abs(l_k - lt) / lt
                assert (rel_l <= tol_l).all(), f"running sum off by {rel_l.max():.3e} (relative)"
            else:
                # the reference trails the max by at most TAU base-2 units and never leads it
                assert (m_k <= mt + tol_m).all() and (m_k >= mt - TAU * LN2 - tol_m).all()
                logsum_k = m_k + np.log(l_k)
                logsum_o = mt + np.log(lt)
                err = np.abs(logsum_k - logsum_o)
                assert (err <= tol_m + tol_l).all(), f"running log-sum off by {err.max():.3e}"
            say(f"  head {b * H + h}: max |dm| {np.abs(m_k - mt).max():.2e}, "
                f"max rel dl {np.abs(l_k * np.exp(m_k - mt) - lt).max() / lt.min():.2e}")
