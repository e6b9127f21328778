"""The backward pass at full size, in the configuration the benchmark times (the
forward ring with its default hand-off and fused fold, then ra_ring_bwd over
the same shards), checked against the fp64 oracle on gradients it can compute
one at a time, and on two identities that hold at any size.

* dq of sampled query rows of the computed ranks (the first and last local row
  of each, token 0 and S-1 when owned, seeded picks): a row needs only its own
  keys.
* dk, dv of every key in the last `tail` tokens, for the listed K/V heads: under
  the causal mask only queries at or after a key see it, so the oracle needs
  lse and D of the computed ranks' rows in that tail only.  The tail spans more
  than one 128-key tile of the local blocks; keys after the last computed query
  must come back exactly zero.
* Summed over all keys, dv equals the sum of dO over the contributing query
  rows (each row's probabilities sum to one), and dk sums to zero (each row's
  dS = P (dP - D) sums to zero, as D = sum_j P dP).  Both are measured against
  the 2-norm over keys of the summed gradient, the size an unconstrained sum of
  those terms would have.  The 16-bit roundings (P or dS into the MFMAs, D from
  the rounded O, the rounded outputs) are unbiased and independent across keys,
  so they move the sum by about 2^-9 of that norm per stage; the bound of 5e-2
  is some 25 times that spread, while a dropped or doubled share of the pairs
  moves it by a sizeable fraction of the norm or more.
"""
import gc
import math

import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import configs, inputs
from long_context_exact_block_amd.pipeline import RingAttention
from tests import parity
from tests.test_gpu_bwd import check_grad
from tests.test_gpu_ring_bwd import REL_MEAN

pytestmark = pytest.mark.gpu

# workload, layout, K/V heads whose tail keys are checked, tail tokens, random dq rows
CASES = [
    (configs.SHARE_1M, "striped", (0, 7), 1536, 48),
    (configs.GQA_128K, "striped", (5,), 1088, 96),
]

SUM_REL = 5e-2  # of the 2-norm over keys, per (batch, K/V head, component)


def _dout(w):
    return inputs.to_dtype(inputs.normal((w.B, w.Hq, w.S, w.d), w.seed + 4), w.dtype)


def ring_grads(w, layout, data, g_st, tag):
    """Forward ring then ra_ring_bwd on the GPU; returns dq, dk, dv (device tensors)."""
    import torch
    tdt = parity.torch_dtype(w.dtype)
    q = parity.to_device(data["q"], w.dtype)
    k = parity.to_device(data["k"], w.dtype)
    v = parity.to_device(data["v"], w.dtype)
    dout = parity.to_device(g_st, w.dtype)
    for key in ("q", "k", "v"):
        del data[key]
    o = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
    lse = torch.zeros((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                       rank0=w.rank0, n_ranks=w.ranks)
    print("%s: forward ring" % tag, flush=True)
    ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()
    dq = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
    dk = torch.zeros((w.B, w.Hkv, w.S, w.d), dtype=tdt, device="cuda")
    dv = torch.zeros((w.B, w.Hkv, w.S, w.d), dtype=tdt, device="cuda")
    print("%s: backward ring" % tag, flush=True)
    ra.backward(dout, dq, dk, dv)
    torch.cuda.synchronize()
    print("%s: backward done" % tag, flush=True)
    del q, k, v, dout, o, lse, ra
    return dq, dk, dv


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,layout,kv_heads,tail,n_rand", CASES,
                         ids=["%s-%s" % (c[0].name, c[1]) for c in CASES])
def test_full_size_backward(w, layout, kv_heads, tail, n_rand):
    check_backward(w, layout, kv_heads, tail, n_rand, ring_grads)


def check_backward(w, layout, kv_heads, tail, n_rand, grads):
    import torch
    assert w.causal, "the tail-key check relies on the causal mask"
    tag = "[full-bwd] %s %s" % (w.name, layout)
    print("\n%s: inputs" % tag, flush=True)
    data = inputs.qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.seed, w.dtype, w.q_scale)
    g_st, g32 = _dout(w)
    dq, dk, dv = grads(w, layout, data, g_st, tag)
    del g_st

    fwd, _ = oracle.layout_maps(rb.LAYOUTS[layout], w.S, w.R)
    owned = np.sort(np.asarray(fwd[w.rank0 * w.n:(w.rank0 + w.ranks) * w.n], np.int64))
    group = w.Hq // w.Hkv
    q32, k32, v32 = data["q32"], data["k32"], data["v32"]

    # --- tail keys: the oracle's rows are the computed ranks' queries in the tail
    t0 = w.S - tail
    tail_rows = owned[owned >= t0]
    rows_b, rows_h, rows_t = [], [], []
    for b in range(w.B):
        for g in kv_heads:
            for h in range(g * group, (g + 1) * group):
                rows_b += [b] * len(tail_rows)
                rows_h += [h] * len(tail_rows)
                rows_t += list(tail_rows)
    n_tail = len(rows_t)
    # --- sampled dq rows anywhere in the sequence
    special, picks = parity.sample_tokens(fwd, w.n, w.rank0, w.ranks, n_rand, seed=w.seed + 9)
    rng = np.random.default_rng(w.seed + 10)
    for t in special:
        rows_b.append(w.B - 1), rows_h.append(w.Hq - 1), rows_t.append(t)
    rows_b += list(rng.integers(0, w.B, len(picks)))
    rows_h += list(rng.integers(0, w.Hq, len(picks)))
    rows_t += list(picks)
    rb_, rh_, rt_ = (np.asarray(x, np.int64) for x in (rows_b, rows_h, rows_t))
    print("%s: oracle dq/lse/D on %d rows (%d tail)" % (tag, len(rt_), n_tail), flush=True)
    rq, rl, rD = oracle.bwd_query_rows(q32[rb_, rh_, rt_], g32[rb_, rh_, rt_], rb_, rh_, rt_,
                                       k32, v32, w.Hq, w.scale, w.causal)
    idx = (torch.from_numpy(rb_), torch.from_numpy(rh_), torch.from_numpy(rt_))
    gq = dq.cpu()[idx].double().numpy()
    rm = REL_MEAN[w.dtype]
    check_grad(gq, rq, tag + " dq rows", rel_mean=rm)
    print("%s: dq rows ok, max err %.3e of max|ref| %.3e" % (
        tag, np.abs(gq - rq).max(), np.abs(rq).max()), flush=True)

    keys = np.arange(t0, w.S, dtype=np.int64)
    kb, kg, kt = (np.asarray(x, np.int64).ravel() for x in np.meshgrid(
        np.arange(w.B), np.asarray(kv_heads), keys, indexing="ij"))
    sl = slice(0, n_tail)
    print("%s: oracle dk/dv on %d keys" % (tag, len(kt)), flush=True)
    rk, rv = oracle.bwd_keys(q32[rb_[sl], rh_[sl], rt_[sl]], g32[rb_[sl], rh_[sl], rt_[sl]],
                             rb_[sl], rh_[sl], rt_[sl], rl[sl], rD[sl], kb, kg, kt, k32, v32,
                             w.Hq, w.scale, w.causal)
    kidx = (torch.from_numpy(kb), torch.from_numpy(kg), torch.from_numpy(kt))
    gk = dk.cpu()[kidx].double().numpy()
    gv = dv.cpu()[kidx].double().numpy()
    check_grad(gk, rk, tag + " dk tail", rel_mean=rm)
    check_grad(gv, rv, tag + " dv tail", rel_mean=rm)
    unseen = kt > owned.max()
    assert not np.any(gk[unseen]) and not np.any(gv[unseen]), "%s: unseen keys not zero" % tag
    print("%s: tail keys ok (%d never seen), dk max err %.3e, dv max err %.3e" % (
        tag, int(unseen.sum()), np.abs(gk - rk).max(), np.abs(gv - rv).max()), flush=True)
    del q32, rq, rk, rv, gq, gk, gv
    data.clear()

    # --- identities over all keys, per (batch, K/V head, component)
    mask = np.zeros(w.S, bool)
    mask[owned] = True
    g_own = g32[:, :, mask].astype(np.float64)
    want_dv = g_own.sum(2).reshape(w.B, w.Hkv, group, w.d).sum(2)
    del g_own, g32
    sum_dv = dv.sum(2, dtype=torch.float64).cpu().numpy()
    sum_dk = dk.sum(2, dtype=torch.float64).cpu().numpy()
    nrm_dv = torch.linalg.vector_norm(dv, dim=2, dtype=torch.float64).cpu().numpy()
    nrm_dk = torch.linalg.vector_norm(dk, dim=2, dtype=torch.float64).cpu().numpy()
    e_dv = np.abs(sum_dv - want_dv) / nrm_dv
    e_dk = np.abs(sum_dk) / nrm_dk
    print("%s: |sum dv - sum dO| %.3e, |sum dk| %.3e (of the 2-norm over keys); "
          "|sum dO| / norm %.1f" % (tag, e_dv.max(), e_dk.max(),
                                    float(np.median(np.abs(want_dv) / nrm_dv))), flush=True)
    assert e_dv.max() <= SUM_REL, "%s: sum_j dv_j off by %.3e" % (tag, e_dv.max())
    assert e_dk.max() <= SUM_REL, "%s: sum_j dk_j off by %.3e" % (tag, e_dk.max())
    del dq, dk, dv
    gc.collect()
    torch.cuda.empty_cache()
    assert math.isfinite(float(rl.sum()))
