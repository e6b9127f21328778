"""Helpers for the GPU parity tests: device upload of seeded inputs, row
sampling, and the tolerance checks (O: max-abs <= 2e-2 and mean-abs <= 2e-3,
LSE: max-abs <= 1e-3, against the fp64 oracle on the same rounded inputs)."""
from __future__ import annotations

import numpy as np

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
# Gradient identities over all keys (full-size backward test): the 16-bit roundings move a sum
# by about 2^-9 of the norm it is measured against per stage; the bound is ~25 times that.
BWD_SUM_REL = 5e-2


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


def bwd_identity_errors(dq, dk, dv, o, q, k, v, dout, group):
    """Two identities of the attention gradients over every row and key, per (batch, K/V head)
    of grouped heads (query head h uses K/V head h // group):
      sum_i <dq_i, q_i> = sum_j <dk_j, k_j>   (both are scale * sum_ij dS_ij <q_i, k_j>),
      sum_j <dv_j, v_j> = sum_i <dO_i, O_i>   (each row's probabilities average its values),
    i over the rows that took part (dq, dO, O zero elsewhere), j over all keys.  Each
    difference is measured against the root sum of squares of the per-row and per-key terms.
    dq, dk, dv, o: torch tensors (any device) [B][H][S][d]; q, k, v, dout: numpy arrays of the
    same shapes.  Returns errors [B][Hkv][2] (the dq/dk identity, the dv/O identity)."""
    import math
    import torch

    def dots(x, y):
        yy = torch.from_numpy(np.ascontiguousarray(y)).to(x.device, torch.float64)
        return (x.double() * yy).sum(-1)

    B, Hkv = dk.shape[0], dk.shape[1]
    out = np.zeros((B, Hkv, 2))
    for b in range(B):
        for g in range(Hkv):
            heads = range(g * group, (g + 1) * group)
            terms = [[dots(dq[b, h], q[b, h]) for h in heads], [dots(dk[b, g], k[b, g])],
                     [dots(dv[b, g], v[b, g])], [dots(o[b, h], dout[b, h]) for h in heads]]
            sums = [float(sum(t.sum() for t in ts)) for ts in terms]
            rss = [math.sqrt(float(sum((t * t).sum() for t in ts))) for ts in terms]
            out[b, g, 0] = abs(sums[0] - sums[1]) / max(rss[0] + rss[1], 1e-300)
            out[b, g, 1] = abs(sums[2] - sums[3]) / max(rss[2] + rss[3], 1e-300)
    return out


def bwd_sum_errors(dk, dv, dout, rows, group):
    """Two sums over all keys, per (batch, K/V head, d component): sum_j dv_j equals the sum of
    dO over the rows that took part (each row's probabilities sum to one), and sum_j dk_j is zero
    (each row's dS sums to zero, as D = sum_j P dP), each against the 2-norm over keys of that
    component of the gradient.  dk, dv: torch tensors (any device) [B][Hkv][S][d]; dout: numpy
    [B][Hq][S][d]; rows: boolean mask over S of the rows that took part.  Returns the largest
    error over components, [B][Hkv][2] (the dv sum, the dk sum)."""
    import torch
    B, Hkv, _, d = dk.shape
    want_dv = dout[:, :, rows].sum(2, dtype=np.float64).reshape(B, Hkv, group, d).sum(2)
    sum_dv = dv.sum(2, dtype=torch.float64).cpu().numpy()
    sum_dk = dk.sum(2, dtype=torch.float64).cpu().numpy()
    nrm_dv = torch.linalg.vector_norm(dv, dim=2, dtype=torch.float64).cpu().numpy()
    nrm_dk = torch.linalg.vector_norm(dk, dim=2, dtype=torch.float64).cpu().numpy()
    out = np.zeros((B, Hkv, 2))
    out[..., 0] = (np.abs(sum_dv - want_dv) / np.maximum(nrm_dv, 1e-300)).max(-1)
    out[..., 1] = (np.abs(sum_dk) / np.maximum(nrm_dk, 1e-300)).max(-1)
    return out
