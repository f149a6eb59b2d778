"""Seeded synthetic inputs shared by the oracle checks, the GPU parity tests and the bench.

This module draws random numbers and rounds them to the storage dtype. It holds
none of the attention arithmetic: no dot products, no softmax, no accumulation.

Recipe (one call per workload):
  * a numpy ``Generator(PCG64(seed))`` draws ``standard_normal`` float32 arrays of
    shape [B, H, N, d], first Q, then K, then V;
  * each array is multiplied by ``mult`` in float32 (the long-sequence stress
    workload uses 3);
  * the float32 values are rounded to the storage dtype with round-to-nearest-even.

The storage-dtype arrays are returned as raw bit patterns so that the CPU oracle
and the GPU path consume exactly the same bits:
  * ``f32``  -> numpy float32
  * ``f16``  -> numpy uint16 holding IEEE binary16 bits
  * ``bf16`` -> numpy uint16 holding bfloat16 bits (the top half of a binary32)
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")
# Integer codes used at the C boundary and by the oracle library.
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), returning uint16 bits.

    Valid for finite inputs, which is all this module produces."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of storage-dtype values (every f16/bf16 value is a float32)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int, mult: float = 1.0):
    """Draw Q, K, V of shape [B, H, N, d] and round them to ``dtype``.

    Returns a dict with keys 'q', 'k', 'v' (storage bits as described above)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[name] = quantize(x, dtype)
        del x
    return out


def make_dout(B: int, H: int, N: int, d: int, seed: int, mult: float = 1.0) -> np.ndarray:
    """Upstream gradient dO of the float32 output O for the backward pass: float32
    [B, H, N, d] drawn iid N(0, 1) (times ``mult``) from ``Generator(PCG64(seed))``.
    Callers pass a seed distinct from the one that drew Q, K, V."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, H, N, d), dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return x


def to_torch(bits: np.ndarray, dtype: str):
    """Wrap storage bits as a torch CPU tensor of the matching dtype (no copy of values)."""
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32))
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
