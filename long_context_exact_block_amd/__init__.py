"""Exact ring attention (one hop = query shard x arriving K/V block, folded
with online softmax) as hand-written HIP kernels for MI355X (gfx950).

The computation lives in libra.so (C ABI in include/ra.h); ``binding`` is the
ctypes layer, ``pipeline`` chains the entry points into one full pass.
"""
from . import binding, configs  # noqa: F401

__all__ = ["binding", "configs"]
