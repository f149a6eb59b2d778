"""Python binding of libfa.so (argument marshalling only).

PyTorch supplies device memory and the stream; every step of the computation runs
in the library's HIP kernels.  The function names follow the C boundary:

    fwd(q, k, v, scale=None)        -> (o, lse)   fused FlashAttention forward
    fwd_split(q, k, v, nsplit=None) -> (o, lse)   the same with each head's keys cut into
                                                  nsplit ranges and merged (few heads)
    naive_fwd(q, k, v, scale=None)  -> (o, lse)   materialised S/P contrast path
    bwd(q, k, v, o, lse, dout)      -> (dq, dk, dv)  backward pass (recomputes P)
    bwd_split(q, k, v, o, lse, dout, nsplit=None)  the same with ranges of rows (few heads)

q, k, v: contiguous [B, H, N, d] device tensors of one dtype (float32, float16 or
bfloat16), d in {64, 128, 256}.  o is float32 [B, H, N, d]; lse is float32 [B, H, N]
(natural log).  scale defaults to 1/sqrt(d).
"""
from __future__ import annotations

import math

import torch

from . import _lib

_CODES = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _CODES:
        raise TypeError("q, k, v must share one dtype among float32, float16, bfloat16")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _on_device(name, t, q):
    """Every caller-supplied buffer must be a tensor on q's device: a host pointer handed
    to a kernel as a device address would fault the GPU."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != q.device:
        raise ValueError(f"{name} must be on {q.device} (got {t.device})")


def _workspace(name, ws, q, nbytes):
    _on_device(name, ws, q)
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"{name} too small: {ws.numel() * ws.element_size()} < {nbytes} bytes")


def _outputs(q, out, lse):
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _on_device("out", out, q)
    _on_device("lse", lse, q)
    if out.dtype != torch.float32 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    if lse.dtype != torch.float32 or lse.shape != q.shape[:3] or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    return out, lse


def _stream(q, stream):
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return ctypes_stream(stream)


def ctypes_stream(stream) -> int:
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream or 0)


def fwd(q, k, v, scale: float | None = None, out=None, lse=None, stream=None):
    """Fused attention forward: returns (o, lse); enqueued on `stream` (default: current)."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    lib = _lib.load()
    rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                    H, N, d, scale, _CODES[q.dtype], _stream(q, stream))
    _lib.check(rc, "fa_fwd")
    return out, lse


def fwd_stats(q, k, v, scale: float | None = None, stream=None):
    """fa_fwd in its statistics-recording form (validation): returns (o, lse, stats) with
    stats float32 [B, H, N, ceil(N/64), 2]: per query row and 64-key block, the kernel's
    running reference (base-2 units) and running row sum after that block."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, None, None)
    stats = torch.empty((B, H, N, (N + 63) // 64, 2), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    rc = lib.fa_fwd_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), stats.data_ptr(), B, H, N, d, scale, _CODES[q.dtype],
                          _stream(q, stream))
    _lib.check(rc, "fa_fwd_stats")
    return out, lse, stats


def split_workspace_bytes(B: int, H: int, N: int, d: int, nsplit: int) -> int:
    return int(_lib.load().fa_fwd_split_workspace_bytes(B, H, N, d, nsplit))


def split_suggest(B: int, H: int, N: int, d: int, compute_units: int) -> int:
    return int(_lib.load().fa_fwd_split_suggest(B, H, N, d, compute_units))


def fwd_split(q, k, v, nsplit: int | None = None, scale: float | None = None, out=None,
              lse=None, workspace=None, stream=None):
    """Key-split fused forward: returns (o, lse), equal to fwd()'s within
    rounding.  nsplit: key ranges per head (default: fa_fwd_split_suggest for the
    device's compute units).  workspace: optional uint8 device tensor of at least
    split_workspace_bytes(B, H, N, d, nsplit) bytes, 256-byte aligned (allocated when
    omitted)."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    if nsplit is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        nsplit = split_suggest(B, H, N, d, cus)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    nbytes = split_workspace_bytes(B, H, N, d, nsplit)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _workspace("split workspace", workspace, q, nbytes)
    lib = _lib.load()
    rc = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), workspace.data_ptr(), int(nsplit), B, H, N, d, scale,
                          _CODES[q.dtype], _stream(q, stream))
    _lib.check(rc, "fa_fwd_split")
    return out, lse


def naive_workspace_bytes(B: int, H: int, N: int, dtype) -> int:
    code = _CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().fa_naive_workspace_bytes(B, H, N, code))


def naive_fwd(q, k, v, scale: float | None = None, out=None, lse=None, workspace=None,
              stream=None):
    """Materialised three-kernel path: returns (o, lse).

    workspace: optional pair of uint8 device tensors (S, P), each at least
    naive_workspace_bytes(B, H, N, dtype) bytes; allocated when omitted."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse)
    nbytes = naive_workspace_bytes(B, H, N, q.dtype)
    if workspace is None:
        workspace = (torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device),
                     torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device))
    s_ws, p_ws = workspace
    _workspace("naive S workspace", s_ws, q, nbytes)
    _workspace("naive P workspace", p_ws, q, nbytes)
    lib = _lib.load()
    rc = lib.fa_naive_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), s_ws.data_ptr(), p_ws.data_ptr(), B, H, N, d, scale,
                          _CODES[q.dtype], _stream(q, stream))
    _lib.check(rc, "fa_naive_fwd")
    return out, lse


def bwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype) -> int:
    code = _CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().fa_bwd_workspace_bytes(B, H, N, d, code))


def bwd(q, k, v, o, lse, dout, scale: float | None = None, workspace=None, grads=None,
        stream=None):
    """Attention backward: returns (dq, dk, dv), float32 tensors shaped like q.

    o and lse are fwd()'s outputs for the same q, k, v and scale; dout is the float32
    gradient of o.  workspace: optional uint8 device tensor of at least
    bwd_workspace_bytes(B, H, N, d, dtype) bytes, 256-byte aligned (allocated when
    omitted).  grads: optional (dq, dk, dv) float32 tensors to write into."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape), ("lse", lse, q.shape[:3])):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.shape != shape
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float32 {tuple(shape)} tensor on {q.device}")
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    for name, t in zip(("dq", "dk", "dv"), grads):
        _on_device(name, t, q)
        if t.dtype != torch.float32 or t.shape != q.shape or not t.is_contiguous():
            raise ValueError("grads must be contiguous float32 tensors shaped like q")
    nbytes = bwd_workspace_bytes(B, H, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _workspace("backward workspace", workspace, q, nbytes)
    lib = _lib.load()
    rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    workspace.data_ptr(), B, H, N, d, scale, _CODES[q.dtype], _stream(q, stream))
    _lib.check(rc, "fa_bwd")
    return dq, dk, dv


def bwd_split_workspace_bytes(B: int, H: int, N: int, d: int, dtype, nsplit: int) -> int:
    code = _CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.load().fa_bwd_split_workspace_bytes(B, H, N, d, code, nsplit))


def bwd_split_suggest(B: int, H: int, N: int, d: int, compute_units: int) -> int:
    return int(_lib.load().fa_bwd_split_suggest(B, H, N, d, compute_units))


def bwd_split(q, k, v, o, lse, dout, nsplit: int | None = None, scale: float | None = None,
              workspace=None, grads=None, stream=None):
    """Backward pass with the key-owned kernel's queries and the query-owned kernel's keys
    cut into ranges whose partial gradients are added: returns (dq, dk, dv)
    like bwd().  nsplit defaults to fa_bwd_split_suggest for the device."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape), ("lse", lse, q.shape[:3])):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.shape != shape
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float32 {tuple(shape)} tensor on {q.device}")
    if nsplit is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        nsplit = bwd_split_suggest(B, H, N, d, cus)
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    for name, t in zip(("dq", "dk", "dv"), grads):
        _on_device(name, t, q)
        if t.dtype != torch.float32 or t.shape != q.shape or not t.is_contiguous():
            raise ValueError("grads must be contiguous float32 tensors shaped like q")
    nbytes = bwd_split_workspace_bytes(B, H, N, d, q.dtype, nsplit)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _workspace("split backward workspace", workspace, q, nbytes)
    lib = _lib.load()
    rc = lib.fa_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), workspace.data_ptr(), int(nsplit), B, H, N, d, scale,
                          _CODES[q.dtype], _stream(q, stream))
    _lib.check(rc, "fa_bwd_split")
    return dq, dk, dv


def version() -> str:
    return _lib.load().fa_version().decode()
