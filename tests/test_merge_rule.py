"""The block-merge rule that fa_fwd_split's merge kernel applies (Triton tutorial section
2.3; the MUSA guide's block update, step e, applied to whole key blocks), checked on the
CPU against the oracle: attention over key ranges, each range's O normalised by its own
row sum and its LSE, merged as
    LSE = log sum_g exp(LSE_g),   O = sum_g exp(LSE_g - LSE) O_g,
equals the oracle's attention over all keys.  The per-range results are computed here
in fp64 numpy from the attention definition; nothing runs on a GPU."""
import numpy as np
import pytest

import oracle
from synth.inputs import make_qkv, to_float32


def range_attention(q, k, v, scale, lo, hi):
    s = scale * np.einsum("bhid,bhjd->bhij", q, k[:, :, lo:hi])
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", e, v[:, :, lo:hi]) / ell
    return o, (m + np.log(ell))[..., 0]


def merge(parts):
    lse = np.stack([p[1] for p in parts])                   # [G, B, H, N]
    m = lse.max(axis=0)
    w = np.exp(lse - m)
    o = sum(w[g][..., None] * parts[g][0] for g in range(len(parts))) / w.sum(axis=0)[..., None]
    return o, m + np.log(w.sum(axis=0))


@pytest.mark.parametrize("dtype,mult,cuts", [
    ("f16", 1.0, [37, 64]),          # uneven ranges
    ("bf16", 3.0, [64]),             # two ranges, wide logits
    ("f16", 8.0, [1, 2, 50, 99]),    # one-key ranges and very wide logits
])
def test_merged_ranges_equal_full_attention(dtype, mult, cuts):
    B, H, N, d = 1, 2, 100, 64
    x = make_qkv(B, H, N, d, dtype, seed=41, mult=mult)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = (to_float32(x[n], dtype).astype(np.float64) for n in ("q", "k", "v"))
    bounds = [0] + cuts + [N]
    parts = [range_attention(q, k, v, scale, lo, hi) for lo, hi in zip(bounds, bounds[1:])]
    o, lse = merge(parts)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], dtype, scale)
    assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert (np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max() <= 1e-12


def test_a_dropped_range_is_caught():
    # the check above is not vacuous: leaving one range out moves O and LSE visibly
    B, H, N, d = 1, 1, 100, 64
    x = make_qkv(B, H, N, d, "f16", seed=42)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = (to_float32(x[n], "f16").astype(np.float64) for n in ("q", "k", "v"))
    parts = [range_attention(q, k, v, scale, lo, hi) for lo, hi in ((0, 40), (40, 100))]
    o, lse = merge(parts[:1])
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], "f16", scale)
    assert np.abs(o - o_ref).max() > 1e-3 and np.abs(lse - lse_ref).max() > 1e-2
