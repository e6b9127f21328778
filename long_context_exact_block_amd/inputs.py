"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle side.

This module holds no attention arithmetic: it only draws N(0,1) samples and
rounds them to the storage dtype.

Recipe (the same for every workload):
* tensor X in {q, k, v} of a workload with seed base ``seed``: the slice
  (b, h) is ``numpy.random.default_rng([seed_X, b, h]).standard_normal((S, d),
  dtype=float32)`` with ``seed_X = seed + {q: 1, k: 2, v: 3}``;
* an optional multiplier (the peaky grouped-query case scales Q by 4, which
  is exact in bf16/fp16);
* round to nearest even into bf16 / fp16 (fp32 is kept as drawn).

The values the GPU receives are returned both as the raw 16-bit storage and as
their exact float32 widening, which is what the oracle reads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_WORKERS = min(16, os.cpu_count() or 1)


def _slice(seed: int, b: int, h: int, rows: int, d: int) -> np.ndarray:
    return np.random.default_rng([seed, b, h]).standard_normal((rows, d), dtype=np.float32)


def normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """float32 tensor [B][H][S][d], slice (b, h) drawn from default_rng([seed, b, h])."""
    B, H, S, d = shape
    out = np.empty((B, H, S, d), np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = _slice(seed, b, h, S, d)
        if scale != 1.0:
            out[b, h] *= np.float32(scale)

    with ThreadPoolExecutor(_WORKERS) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 storage."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(
        np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(x: np.ndarray, dtype: str):
    """Return (storage array, exact float32 widening) for dtype in {bf16, fp16, fp32}."""
    if dtype == "fp32":
        x = np.ascontiguousarray(x, np.float32)
        return x, x
    if dtype == "bf16":
        bits = round_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    if dtype == "fp16":
        h = np.ascontiguousarray(x, np.float32).astype(np.float16)
        return h, h.astype(np.float32)
    raise ValueError(dtype)


def qkv(B: int, Hq: int, Hkv: int, S: int, d: int, seed: int, dtype: str, q_scale: float = 1.0):
    """Q [B][Hq][S][d], K, V [B][Hkv][S][d] in the original token order.

    Returns dict with 'q', 'k', 'v' (storage arrays) and 'q32', 'k32', 'v32'
    (exact float32 values of the same numbers).
    """
    out = {}
    for name, off, H, sc in (("q", 1, Hq, q_scale), ("k", 2, Hkv, 1.0), ("v", 3, Hkv, 1.0)):
        x = normal((B, H, S, d), seed + off, sc)
        st, f = to_dtype(x, dtype)
        del x
        out[name] = st
        out[name + "32"] = f
    return out
