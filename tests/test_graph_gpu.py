"""The library under HIP graph capture: the forward (persistent forms at d = 128 and 256,
the per-tile form at d = 64), the key-split forward (with a workspace and in its
allocation-free form) and the backward, each captured once on a side stream and replayed
three times.  Between the replays the program clears the outputs and runs eager work of
its own, with synchronizations; every replay must reproduce the eager call bitwise.  The
library issues no allocation, memset or synchronization, so nothing of it needs to stay
out of the graph."""
import math

import pytest
import torch

import exact_attention_90_amd as fa
from exact_attention_90_amd import _lib
from synth.inputs import make_qkv
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def _replay_matches(g, outs, refs, name):
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        noise = torch.randn(1 << 16, device="cuda")  # eager work between the replays
        (noise * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), f"{name}: replay {rep} differs from the eager call"


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # once outside the graph on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("B,H,N,d,dtype", [(1, 300, 256, 128, "bf16"), (1, 300, 128, 256, "bf16"),
                                          (2, 4, 512, 64, "f16")])
def test_forward_replays(B, H, N, d, dtype):
    xd = to_device(make_qkv(B, H, N, d, dtype, seed=40 + d), dtype)
    scale = 1.0 / math.sqrt(d)
    say(f"graph fwd B={B} H={H} N={N} d={d} {dtype}")
    o_ref, lse_ref = fa.fwd(xd["q"], xd["k"], xd["v"], scale)
    out, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    g = _capture(lambda: fa.fwd(xd["q"], xd["k"], xd["v"], scale, out=out, lse=lse))
    _replay_matches(g, (out, lse), (o_ref, lse_ref), "fa_fwd")


def test_split_forward_replays():
    B, H, N, d, dtype, nsplit = 1, 2, 4096, 128, "bf16", 4
    xd = to_device(make_qkv(B, H, N, d, dtype, seed=44), dtype)
    q, k, v = xd["q"], xd["k"], xd["v"]
    scale = 1.0 / math.sqrt(d)
    say("graph fwd_split and fa_fwd_split_noalloc")
    ws = torch.empty(fa.split_workspace_bytes(B, H, N, d, nsplit), dtype=torch.uint8, device="cuda")
    o_ref, lse_ref = fa.fwd_split(q, k, v, nsplit, scale, workspace=ws)
    out, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    g = _capture(lambda: fa.fwd_split(q, k, v, nsplit, scale, out=out, lse=lse, workspace=ws))
    _replay_matches(g, (out, lse), (o_ref, lse_ref), "fa_fwd_split")

    lib = _lib.load()
    out2, lse2 = torch.empty_like(o_ref), torch.empty_like(lse_ref)

    def noalloc():
        rc = lib.fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out2.data_ptr(),
                                      lse2.data_ptr(), nsplit, B, H, N, d, scale, _lib.FA_BF16,
                                      torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc

    g2 = _capture(noalloc)
    _replay_matches(g2, (out2, lse2), (o_ref, lse_ref), "fa_fwd_split_noalloc")


def test_backward_replays():
    B, H, N, d, dtype = 1, 8, 512, 128, "bf16"
    xd = to_device(make_qkv(B, H, N, d, dtype, seed=45), dtype)
    q, k, v = xd["q"], xd["k"], xd["v"]
    scale = 1.0 / math.sqrt(d)
    say("graph bwd")
    o, lse = fa.fwd(q, k, v, scale)
    dout = torch.randn(q.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(5))
    ws = torch.empty(max(fa.bwd_workspace_bytes(B, H, N, d, q.dtype), 256), dtype=torch.uint8,
                     device="cuda")
    refs = fa.bwd(q, k, v, o, lse, dout, scale, workspace=ws)
    grads = tuple(torch.empty_like(r) for r in refs)
    g = _capture(lambda: fa.bwd(q, k, v, o, lse, dout, scale, workspace=ws, grads=grads))
    _replay_matches(g, grads, refs, "fa_bwd")
