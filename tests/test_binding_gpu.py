"""The Python binding refuses buffers that are not on the inputs' device before anything
is enqueued: a host pointer passed to a kernel as a device address would fault the GPU.
Every check here raises on the host; no kernel is launched with a bad buffer."""
import pytest
import torch

import exact_attention_90_amd as fa
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

B, H, N, d = 1, 2, 70, 64


@pytest.fixture(scope="module")
def qkv():
    g = torch.Generator().manual_seed(5)
    return tuple(torch.randn((B, H, N, d), generator=g).to(torch.float16).cuda() for _ in range(3))


def _host(shape, dtype=torch.float32):
    return torch.empty(shape, dtype=dtype)


def test_fwd_rejects_host_outputs(qkv):
    say("binding: fwd with host out / lse")
    q, k, v = qkv
    with pytest.raises(ValueError, match="out must be on"):
        fa.fwd(q, k, v, out=_host(q.shape))
    with pytest.raises(ValueError, match="lse must be on"):
        fa.fwd(q, k, v, lse=_host(q.shape[:3]))
    with pytest.raises(TypeError, match="out must be a torch.Tensor"):
        fa.fwd(q, k, v, out=[0.0])


def test_split_and_naive_reject_host_workspace(qkv):
    say("binding: fwd_split / naive_fwd with host workspace")
    q, k, v = qkv
    nbytes = fa.split_workspace_bytes(B, H, N, d, 2)
    with pytest.raises(ValueError, match="split workspace must be on"):
        fa.fwd_split(q, k, v, 2, workspace=_host((nbytes,), torch.uint8))
    nb = fa.naive_workspace_bytes(B, H, N, q.dtype)
    dev = torch.empty(nb, dtype=torch.uint8, device=q.device)
    with pytest.raises(ValueError, match="naive S workspace must be on"):
        fa.naive_fwd(q, k, v, workspace=(_host((nb,), torch.uint8), dev))
    with pytest.raises(ValueError, match="naive P workspace must be on"):
        fa.naive_fwd(q, k, v, workspace=(dev, _host((nb,), torch.uint8)))


def test_bwd_rejects_host_grads_and_workspace(qkv):
    say("binding: bwd / bwd_split with host grads or workspace")
    q, k, v = qkv
    o, lse = fa.fwd(q, k, v)
    dout = torch.ones_like(o)
    dev_grads = [torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3)]
    for i, name in enumerate(("dq", "dk", "dv")):
        grads = list(dev_grads)
        grads[i] = _host(q.shape)
        with pytest.raises(ValueError, match=f"{name} must be on"):
            fa.bwd(q, k, v, o, lse, dout, grads=tuple(grads))
        with pytest.raises(ValueError, match=f"{name} must be on"):
            fa.bwd_split(q, k, v, o, lse, dout, 2, grads=tuple(grads))
    nb = fa.bwd_workspace_bytes(B, H, N, d, q.dtype)
    with pytest.raises(ValueError, match="backward workspace must be on"):
        fa.bwd(q, k, v, o, lse, dout, workspace=_host((nb,), torch.uint8))
    nb = fa.bwd_split_workspace_bytes(B, H, N, d, q.dtype, 2)
    with pytest.raises(ValueError, match="split backward workspace must be on"):
        fa.bwd_split(q, k, v, o, lse, dout, 2, workspace=_host((nb,), torch.uint8))
    with pytest.raises(ValueError, match="dout must be a contiguous float32"):
        fa.bwd(q, k, v, o, lse, dout.cpu())
    torch.cuda.synchronize()
