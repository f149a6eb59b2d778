"""fa_fwd_split_noalloc, the key-split forward without a workspace argument (its partials
live in the library's static device scratch), called through the C boundary and checked
against fa_fwd_split on the same inputs: two calls in a row, the second smaller, then a
problem too large for the scratch, which must be refused before anything is enqueued."""
import math

import numpy as np
import pytest
import torch

from exact_attention_90_amd import _lib
from synth.inputs import make_qkv, to_torch
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

CODES = {"f32": _lib.FA_F32, "f16": _lib.FA_F16, "bf16": _lib.FA_BF16}


def _call_pair(B, H, N, d, dtype, nsplit, seed):
    lib = _lib.load()
    x = make_qkv(B, H, N, d, dtype, seed)
    q, k, v = (to_torch(x[n], dtype).cuda() for n in "qkv")
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = lib.fa_fwd_split_workspace_bytes(B, H, N, d, nsplit)
    assert 0 < nbytes <= _lib.FA_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for name in ("fa_fwd_split", "fa_fwd_split_noalloc"):
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        say(f"{name} B={B} H={H} N={N} d={d} {dtype} nsplit={nsplit}")
        if name == "fa_fwd_split":
            rc = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), ws.data_ptr(), nsplit, B, H, N, d, scale,
                                  CODES[dtype], stream)
        else:
            rc = lib.fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), nsplit, B, H, N, d, scale,
                                          CODES[dtype], stream)
        assert rc == 0, (name, rc, lib.fa_status_string(rc))
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.isfinite(o2).all() and torch.isfinite(l2).all()
    # the same kernels on the same inputs: bitwise equal, hence within every tolerance
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert float((o1 - o2).abs().max()) <= tol


def test_noalloc_matches_fa_fwd_split_twice():
    # a larger problem first, then a smaller one: the second call must not see the
    # first call's partials left in the scratch
    _call_pair(1, 2, 3000, 128, "bf16", 4, seed=21)
    _call_pair(1, 1, 1000, 64, "f16", 3, seed=22)
    _call_pair(2, 1, 200, 64, "f32", 2, seed=23)


def test_noalloc_refuses_more_than_the_scratch():
    lib = _lib.load()
    B, H, N, d, nsplit = 1, 8, 8192, 128, 4
    assert lib.fa_fwd_split_workspace_bytes(B, H, N, d, nsplit) > _lib.FA_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, H, N, d), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), 7.0, dtype=torch.float32, device="cuda")
    say("fa_fwd_split_noalloc beyond the scratch")
    rc = lib.fa_fwd_split_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), nsplit, B, H, N, d, 0.1, _lib.FA_BF16,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 9 and _lib.STATUS[rc] == "FA_ERR_SCRATCH"
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())  # nothing was written
