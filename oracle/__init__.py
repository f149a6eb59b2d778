"""CPU fp64 oracle for the attention forward pass (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline
leg may use it; the product path never does.  It shares no code with the GPU
library.

What it computes (MUSA SDK guide "FlashAttention optimization", sections on the
standard three-step attention and safe softmax; pwwt.cn Triton tutorial,
sections 1 and 2.3): for every query row, s = scale * q K^T, P = softmax(s) with
the row max subtracted, o = P V, and LSE = m + ln(sum exp(s - m)).

``online_head`` runs the blockwise online-softmax recurrences of the MUSA guide's
FlashAttention formula (steps 1-4, a-f) and records (m, l) after every block.

``attention_bwd`` gives dQ, dK, dV for an upstream gradient dO: the chain rule of
O = softmax(scale Q K^T) V with P recomputed (Triton tutorial, sections 2.4 and 4.4),
written out in the C source.

Inputs are storage bits as produced by ``synth.inputs`` (float32 arrays, or uint16
bit patterns for f16/bf16); they are widened exactly to double inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_attention.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, I64, ctypes.c_double,
                                     P, I64, P, P]
    lib.oracle_head_steps.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, I64,
                                      ctypes.c_double, I64, P, P, P, P]
    lib.oracle_online_head.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, I64,
                                       ctypes.c_double, I64, I64, P, P, P, P]
    lib.oracle_attention_bwd.argtypes = [P, P, P, P, ctypes.c_int, I64, I64, I64, I64,
                                         ctypes.c_double, P, I64, P, P, P]
    for f in (lib.oracle_attention, lib.oracle_head_steps, lib.oracle_online_head,
              lib.oracle_attention_bwd):
        f.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def use_library(path):
    """Point this module at another build of oracle.c (used by the mutation test).
    Returns the previously loaded library handle (or None)."""
    global _lib
    prev = _lib
    _lib = _configure(ctypes.CDLL(path)) if path is not None else None
    return prev


def restore_library(handle):
    global _lib
    _lib = handle


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _prep(q, k, v, dtype):
    if dtype not in _CODES:
        raise ValueError(f"unknown dtype {dtype!r}")
    want = np.float32 if dtype == "f32" else np.uint16
    arrs = []
    for a in (q, k, v):
        a = np.ascontiguousarray(a)
        if a.dtype != want:
            raise TypeError(f"{dtype} inputs must be {np.dtype(want).name} arrays, got {a.dtype}")
        arrs.append(a)
    if not (arrs[0].shape == arrs[1].shape == arrs[2].shape) or arrs[0].ndim != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    return arrs


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def attention(q, k, v, dtype: str, scale: float, rows=None):
    """Oracle O and LSE.

    rows: None for every row (O has shape [B, H, N, d], LSE [B, H, N]), or an
    int array of global row indices (b*H + h)*N + i, in which case O is
    [len(rows), d] and LSE [len(rows)], in the order given."""
    q, k, v = _prep(q, k, v, dtype)
    B, H, N, d = q.shape
    lib = _load()
    if rows is None:
        o = np.empty((B, H, N, d), np.float64)
        lse = np.empty((B, H, N), np.float64)
        rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _CODES[dtype], B, H, N, d,
                                  float(scale), None, 0, _ptr(o), _ptr(lse))
        if rc:
            raise RuntimeError(f"oracle_attention failed ({rc})")
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).ravel()
    order = np.argsort(rows, kind="stable")
    srows = np.ascontiguousarray(rows[order])
    o_s = np.empty((len(rows), d), np.float64)
    lse_s = np.empty((len(rows),), np.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _CODES[dtype], B, H, N, d, float(scale),
                              _ptr(srows), len(srows), _ptr(o_s), _ptr(lse_s))
    if rc:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    o = np.empty_like(o_s)
    lse = np.empty_like(lse_s)
    o[order] = o_s
    lse[order] = lse_s
    return o, lse


def head_steps(q, k, v, dtype: str, scale: float, head: int = 0):
    """S, P, O, LSE of one head (head = b*H + h) through the three standard steps."""
    q, k, v = _prep(q, k, v, dtype)
    B, H, N, d = q.shape
    s = np.empty((N, N), np.float64)
    p = np.empty((N, N), np.float64)
    o = np.empty((N, d), np.float64)
    lse = np.empty((N,), np.float64)
    rc = _load().oracle_head_steps(_ptr(q), _ptr(k), _ptr(v), _CODES[dtype], B, H, N, d,
                                   float(scale), head, _ptr(s), _ptr(p), _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError(f"oracle_head_steps failed ({rc})")
    return s, p, o, lse


def online_head(q, k, v, dtype: str, scale: float, block: int, head: int = 0):
    """Blockwise online softmax of one head: (O, LSE, m_trace, l_trace)."""
    q, k, v = _prep(q, k, v, dtype)
    B, H, N, d = q.shape
    nb = (N + block - 1) // block
    o = np.empty((N, d), np.float64)
    lse = np.empty((N,), np.float64)
    mt = np.empty((N, nb), np.float64)
    lt = np.empty((N, nb), np.float64)
    rc = _load().oracle_online_head(_ptr(q), _ptr(k), _ptr(v), _CODES[dtype], B, H, N, d,
                                    float(scale), head, block, _ptr(o), _ptr(lse), _ptr(mt),
                                    _ptr(lt))
    if rc:
        raise RuntimeError(f"oracle_online_head failed ({rc})")
    return o, lse, mt, lt


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def attention_bwd(q, k, v, dout, dtype: str, scale: float, heads=None):
    """Oracle gradients (dq, dk, dv) of O with respect to Q, K, V for the upstream
    gradient dout (float32 [B, H, N, d]).  heads: None for every head (outputs
    [B, H, N, d]) or ascending head indices b*H + h (outputs [len(heads), N, d])."""
    q, k, v = _prep(q, k, v, dtype)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    if dout.shape != q.shape:
        raise ValueError("dout must have the [B, H, N, d] shape of q")
    B, H, N, d = q.shape
    lib = _load()
    if heads is None:
        shape, hp, nh = (B, H, N, d), None, B * H
    else:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int64).ravel())
        shape, hp, nh = (len(hs), N, d), _ptr(hs), len(hs)
    dq, dk, dv = (np.empty(shape, np.float64) for _ in range(3))
    rc = lib.oracle_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _CODES[dtype], B, H, N,
                                  d, float(scale), hp, nh, _ptr(dq), _ptr(dk), _ptr(dv))
    if rc:
        raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
    return dq, dk, dv
