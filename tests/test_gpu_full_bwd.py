"""The backward pass at full size, in the configuration the benchmark times (the
forward ring with its default hand-off and fused fold, then ra_ring_bwd over
the same shards), checked against the fp64 oracle on gradients it can compute
one at a time, and on identities that hold at any size.

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
* Over every row and key, sum_i <dq_i, q_i> = sum_j <dk_j, k_j> (both are
  scale * sum_ij dS_ij <q_i, k_j>) and sum_j <dv_j, v_j> = sum_i <dO_i, O_i>
  (each row's probabilities average its values), per batch and K/V head, with
  the same bound against the root sum of squares of the per-row and per-key
  terms: they tie the dq kernel to the dk kernel, and dv to the forward output,
  on every key rather than the tail only.
* The per-hop unit itself (ra_block_bwd) at the 1M share's hop shape, and the whole
  ring backward on the 1M share: both take lse and O as inputs, so with seeded
  stand-ins on both sides the oracle computes dk and dv of keys anywhere -- in the
  131,072-key block (both striped block classes), and over the whole 1,048,576-token
  sequence through the ring's dk/dv hand-off.
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

SUM_REL = parity.BWD_SUM_REL  # of the 2-norm over keys, per (batch, K/V head, component)


def _dout(w):
    return inputs.to_dtype(inputs.normal((w.B, w.Hq, w.S, w.d), w.seed + 4), w.dtype)


def ring_grads(w, layout, data, g_st, tag):
    """Forward ring then ra_ring_bwd on the GPU; returns dq, dk, dv and the forward's O
    (device tensors)."""
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
    del q, k, v, dout, lse, ra
    return dq, dk, dv, o


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
    dq, dk, dv, o = grads(w, layout, data, g_st, tag)
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
    del rq, rk, rv, gq, gk, gv

    # --- inner-product identities over every row and key, per (batch, K/V head):
    #   sum_i <dq_i, q_i> = sum_j <dk_j, k_j>  (both are scale * sum_ij dS_ij <q_i, k_j>),
    #   sum_j <dv_j, v_j> = sum_i <dO_i, O_i>  (each row's probabilities average its values),
    # i over the computed ranks' rows of the group's query heads, j over all keys.  They tie
    # the dq kernel to the dk kernel and dv to the forward output on every key, not only the
    # tail.  Measured against the root sum of squares of the per-row / per-key terms: the
    # 16-bit roundings move each term by about 2^-9 of itself, independently.
    errs = parity.bwd_identity_errors(dq, dk, dv, o, q32, k32, v32, g32, group)
    worst = errs.max(axis=(0, 1))
    assert worst[0] <= SUM_REL, "%s: sum <dq,q> vs sum <dk,k> off by %.3e" % (tag, worst[0])
    assert worst[1] <= SUM_REL, "%s: sum <dv,v> vs sum <dO,O> off by %.3e" % (tag, worst[1])
    print("%s: |sum<dq,q> - sum<dk,k>| %.3e, |sum<dv,v> - sum<dO,O>| %.3e (of the root sum of "
          "squares of the terms)" % (tag, worst[0], worst[1]), flush=True)
    del q32, o
    data.clear()

    # --- sums over all keys, per (batch, K/V head, component)
    mask = np.zeros(w.S, bool)
    mask[owned] = True
    errs = parity.bwd_sum_errors(dk, dv, g32, mask, group)
    del g32
    e_dv, e_dk = errs[..., 0].max(), errs[..., 1].max()
    print("%s: |sum dv - sum dO| %.3e, |sum dk| %.3e (of the 2-norm over keys)" % (
        tag, e_dv, e_dk), flush=True)
    assert e_dv <= SUM_REL, "%s: sum_j dv_j off by %.3e" % (tag, e_dv)
    assert e_dk <= SUM_REL, "%s: sum_j dk_j off by %.3e" % (tag, e_dk)
    del dq, dk, dv
    gc.collect()
    torch.cuda.empty_cache()
    assert math.isfinite(float(rl.sum()))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kg0,shift", [(3, 0), (4, 1)], ids=["src_le_rank", "src_gt_rank"])
def test_block_bwd_full_hop_keys_everywhere(kg0, shift):
    """ra_block_bwd at the 1M-token share's per-hop shape (131,072 queries x 131,072 keys,
    d = 128, bf16, one head) in both striped block classes of rank 3: query ids 3 + 8i and
    key ids kg0 + 8j, so key j is allowed for query i iff j <= i (a source at or below the
    rank, kg0 = 3) or j < i (above it, kg0 = 4).  dk and dv are compared element by element
    at keys spread over the whole block -- key 0, which (nearly) every query sees, tile and
    workgroup boundaries, seeded picks and the last keys.  The block kernels take lse and O
    as inputs, so both sides get the same seeded stand-ins: lse_i = ln(#allowed keys) +
    scale^2 |q_i|^2 / 2 (what ln sum_j exp(s_ij) is for Gaussian scores, so the
    probabilities have their real scale), O and dO seeded, and the oracle needs no forward
    pass over the block.  It sees the block as a causal sequence of its own: row i at
    position i, key j at position j + shift."""
    import torch
    n, d = 131072, 128
    scale = 1.0 / math.sqrt(d)
    shp = (1, 1, n, d)
    q_st, q32 = inputs.to_dtype(inputs.normal(shp, 7101), "bf16")
    k_st, k32 = inputs.to_dtype(inputs.normal(shp, 7102), "bf16")
    v_st, v32 = inputs.to_dtype(inputs.normal(shp, 7103), "bf16")
    g_st, g32 = inputs.to_dtype(inputs.normal(shp, 7104), "bf16")
    o_st, o32 = inputs.to_dtype(0.05 * inputs.normal(shp, 7105), "bf16")
    qd = q32[0, 0].astype(np.float64)
    allowed = np.maximum(np.arange(1, n + 1, dtype=np.float64) - shift, 1.0)
    lse = np.log(allowed) + 0.5 * scale * scale * (qd * qd).sum(-1)
    lse = lse.astype(np.float32).astype(np.float64)  # the kernel reads it as fp32
    Dv = (g32[0, 0].astype(np.float64) * o32[0, 0].astype(np.float64)).sum(-1)

    dev = lambda st: parity.to_device(st, "bf16")
    q, k, v, g, o = dev(q_st), dev(k_st), dev(v_st), dev(g_st), dev(o_st)
    lse_d = torch.from_numpy(lse.astype(np.float32).reshape(1, 1, n)).cuda()
    dq = torch.zeros(shp, dtype=torch.float32, device="cuda")
    dk = torch.zeros(shp, dtype=torch.float32, device="cuda")
    dv = torch.zeros(shp, dtype=torch.float32, device="cuda")
    a = rb.block_bwd_args(q, k, v, o, g, lse_d, dq, dk, dv, scale, True, 3, 8, kg0, 8)
    ws = torch.empty(max(rb.ra_block_bwd_workspace_size(a), 256), dtype=torch.uint8,
                     device="cuda")
    print("\n[block-bwd full hop kg0=%d] kernels" % kg0, flush=True)
    rb.ra_block_bwd(a, ws)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7106 + kg0)
    keys = np.unique(np.concatenate([
        [0, 1, 31, 32, 63, 64, 255, 256, 257, 4095, 4096, n // 2, n - 257, n - 256, n - 2,
         n - 1], rng.integers(0, n, 112)])).astype(np.int64)
    rows = np.arange(n, dtype=np.int64)
    zeros = np.zeros(n, np.int64)
    kz = np.zeros(len(keys), np.int64)
    k_seq, v_seq = k32, v32
    if shift:  # key j at position j + 1: a leading row no query is paired with first
        pad = np.zeros((1, 1, shift, d), np.float32)
        k_seq = np.concatenate([pad, k32], axis=2)
        v_seq = np.concatenate([pad, v32], axis=2)
    print("[block-bwd full hop kg0=%d] oracle dk/dv on %d keys" % (kg0, len(keys)), flush=True)
    rk, rv = oracle.bwd_keys(q32[0, 0], g32[0, 0], zeros, zeros, rows, lse, Dv, kz, kz,
                             keys + shift, k_seq, v_seq, 1, scale, True)
    gk = dk[0, 0].cpu().numpy().astype(np.float64)[keys]
    gv = dv[0, 0].cpu().numpy().astype(np.float64)[keys]
    check_grad(gk, rk, "full hop block dk kg0=%d" % kg0)
    check_grad(gv, rv, "full hop block dv kg0=%d" % kg0)
    if shift:  # the last key is allowed for no query of a block above the rank
        assert not np.any(gk[keys == n - 1]) and not np.any(gv[keys == n - 1])
    print("[block-bwd full hop kg0=%d] dk max err %.3e of max|ref| %.3e, dv max err %.3e of "
          "%.3e" % (kg0, np.abs(gk - rk).max(), np.abs(rk).max(), np.abs(gv - rv).max(),
                    np.abs(rv).max()), flush=True)
    del q, k, v, g, o, dq, dk, dv, ws
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [configs.SHARE_1M, configs.GQA_128K], ids=lambda w: w.name)
def test_ring_bwd_keys_everywhere(w):
    """ra_ring_bwd at full size (the 1M-token share, rank 3 of 8; the peaky 128k GQA ring,
    all 8 ranks, four query heads per K/V head; striped, bf16, COPY hand-off: K, V and the
    dk/dv accumulators travel around the ring) with dk and dv compared element by element
    at keys all over the sequence -- token 0, block and tile boundaries, seeded picks in
    every K/V head, and the last tokens (on the 1M share no query of rank 3 sees them).
    The backward takes the forward's O and lse as inputs, so both sides get seeded
    stand-ins for the computed rows (lse_t = ln(t + 1) + scale^2 |q_t|^2 / 2: the size of
    ln sum_j exp(s_tj) for Gaussian scores of moderate spread over the t + 1 allowed keys;
    under the x4 logits of the peaky workload it falls short of the true value, so some
    probabilities exceed 1 and the gradients are larger, alike on both sides; O seeded) and
    the oracle needs no forward pass over the sequence."""
    import torch
    assert w.B == 1 and w.causal
    tag = "[ring-bwd keys everywhere %s]" % w.name
    print("\n%s inputs" % tag, flush=True)
    data = inputs.qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.seed, w.dtype, w.q_scale)
    g_st, g32 = _dout(w)
    o_st, o32 = inputs.to_dtype(0.05 * inputs.normal((w.B, w.Hq, w.S, w.d), w.seed + 11),
                                w.dtype)
    tdt = parity.torch_dtype(w.dtype)
    q = parity.to_device(data["q"], w.dtype)
    k = parity.to_device(data["k"], w.dtype)
    v = parity.to_device(data["v"], w.dtype)
    o = parity.to_device(o_st, w.dtype)
    dout = parity.to_device(g_st, w.dtype)
    for key in ("q", "k", "v"):
        del data[key]
    del o_st, g_st
    ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, "striped", tdt, w.causal, w.scale,
                       rank0=w.rank0, n_ranks=w.ranks, handoff=rb.HANDOFF_COPY)
    ra.maps()
    ra.gather(q, k, v)
    rb.ra_layout_gather(o, ra.o_sh, ra.fwd, w.R, w.rank0, w.ranks)
    fwd, _ = oracle.layout_maps(rb.LAYOUTS["striped"], w.S, w.R)
    # slot -> token of the computed ranks' local rows, [ranks][n]
    toks = np.asarray(fwd[w.rank0 * w.n:(w.rank0 + w.ranks) * w.n], np.int64).reshape(
        w.ranks, w.n)
    q32 = data["q32"]
    qq = np.einsum("hrnd,hrnd->hrn", q32[0][:, toks], q32[0][:, toks])  # [Hq][ranks][n]
    lse = (np.log(toks + 1.0)[None] + 0.5 * w.scale * w.scale * qq).astype(np.float32)
    ra.lse_sh.copy_(torch.from_numpy(np.ascontiguousarray(lse.transpose(1, 0, 2))).reshape(
        ra.lse_sh.shape))
    dq = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
    dk = torch.zeros((w.B, w.Hkv, w.S, w.d), dtype=tdt, device="cuda")
    dv = torch.zeros((w.B, w.Hkv, w.S, w.d), dtype=tdt, device="cuda")
    print("%s backward ring" % tag, flush=True)
    ra.backward(dout, dq, dk, dv)
    torch.cuda.synchronize()
    del q, k, v, o, dout, ra, dq

    rng = np.random.default_rng(w.seed + 12)
    n = w.n
    fixed = np.array([0, 1, 2, 3, 4, 7, 8, 11, 255, 256, 2047, 2048, n - 1, n, n + 1,
                      w.S // 2, w.S - 5, w.S - 4, w.S - 1], np.int64)
    kb, kg, kt = [], [], []
    for g in range(w.Hkv):
        tk = np.unique(np.concatenate([fixed, rng.integers(0, w.S, 14)]))
        kg += [g] * len(tk)
        kt += list(tk)
        kb += [0] * len(tk)
    kb, kg, kt = (np.asarray(x, np.int64) for x in (kb, kg, kt))
    flat = toks.reshape(-1)
    rows_h = np.repeat(np.arange(w.Hq, dtype=np.int64), flat.size)
    rows_t = np.tile(flat, w.Hq)
    rows_b = np.zeros_like(rows_t)
    q_rows = q32[0][rows_h, rows_t]
    g_rows = g32[0][rows_h, rows_t]
    Dv = (g_rows.astype(np.float64) * o32[0][rows_h, rows_t].astype(np.float64)).sum(-1)
    lse_rows = lse.reshape(-1).astype(np.float64)  # [Hq][ranks][n], as the rows
    print("%s oracle dk/dv on %d keys from %d rows" % (tag, len(kt), len(rows_t)), flush=True)
    rk, rv = oracle.bwd_keys(q_rows, g_rows, rows_b, rows_h, rows_t, lse_rows, Dv, kb, kg, kt,
                             data["k32"], data["v32"], w.Hq, w.scale, w.causal)
    idx = (torch.from_numpy(kb), torch.from_numpy(kg), torch.from_numpy(kt))
    gk = dk.cpu()[idx].double().numpy()
    gv = dv.cpu()[idx].double().numpy()
    rm = REL_MEAN[w.dtype]
    check_grad(gk, rk, tag + " dk", rel_mean=rm)
    check_grad(gv, rv, tag + " dv", rel_mean=rm)
    unseen = kt > flat.max()
    assert not np.any(gk[unseen]) and not np.any(gv[unseen])
    if w.ranks < w.R:
        assert unseen.any()
    print("%s dk max err %.3e of max|ref| %.3e, dv max err %.3e of %.3e (%d keys unseen)" % (
        tag, np.abs(gk - rk).max(), np.abs(rk).max(), np.abs(gv - rv).max(), np.abs(rv).max(),
        int(unseen.sum())), flush=True)
    del dk, dv
    data.clear()
    gc.collect()
    torch.cuda.empty_cache()
