"""Helpers for the GPU parity tests: device upload of seeded inputs, row
sampling, and the tolerance checks (O: max-abs <= 2e-2 and mean-abs <= 2e-3,
LSE: max-abs <= 1e-3, against the fp64 oracle on the same rounded inputs)."""
from __future__ import annotations

import numpy as np

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[name]


def to_device(storage, dtype_name):
    """numpy storage (uint16 bf16 bits / float16 / float32) -> CUDA tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(storage))
    if dtype_name == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def to_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_o(o_gpu, o_ref, what=""):
    err = np.abs(np.asarray(o_gpu, np.float64) - np.asarray(o_ref, np.float64))
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert np.isfinite(err).all(), "%s: non-finite O" % what
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, "%s: O max %.3e mean %.3e" % (what, mx, mean)
    return mx, mean


def check_lse(lse_gpu, lse_ref, what=""):
    a = np.asarray(lse_gpu, np.float64)
    b = np.asarray(lse_ref, np.float64)
    both_inf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    mx = float(err.max()) if err.size else 0.0
    assert np.isfinite(err).all() and mx <= LSE_MAX_ABS, "%s: LSE max %.3e" % (what, mx)
    return mx


def sample_tokens(fwd, n, rank0, n_ranks, count, seed):
    """Global tokens owned by the computed ranks: token 0 and S-1 when owned,
    the first and last local row of every computed rank (under the striped
    layout the first local row is the one with no key in blocks from higher
    ranks), plus `count` seeded picks spread evenly over the eight 32-row
    wave slots of a 256-row workgroup."""
    owned = np.asarray(fwd[rank0 * n:(rank0 + n_ranks) * n], np.int64)
    S = len(fwd)
    special = set()
    owned_set = None
    for t in (0, S - 1):
        if owned_set is None:
            owned_set = set(owned.tolist()) if owned.size < 5_000_000 else None
        if owned_set is not None and t in owned_set:
            special.add(t)
    for r in range(rank0, rank0 + n_ranks):
        special.add(int(fwd[r * n]))
        special.add(int(fwd[r * n + n - 1]))
    # picks spread evenly over the eight 32-row wave slots of the kernels' 256-row
    # workgroups (the waves that lead and lag within a tile), by local row index
    rng = np.random.default_rng(seed)
    slot = (np.arange(owned.size) % n) % 256 // 32
    picks = []
    for c in range(8):
        pool = owned[slot == c]
        take = min(pool.size, count // 8 + (1 if c < count % 8 else 0))
        if take:
            picks.extend(rng.choice(pool, size=take, replace=False).tolist())
    return sorted(special), np.asarray(picks, np.int64)
