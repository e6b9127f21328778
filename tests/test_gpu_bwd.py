"""ra_block_bwd (gradient contributions of one query shard x one K/V block)
against the fp64 oracle's block backward on the same rounded inputs: several
tiles, ragged tails, both layouts' masks, grouped heads, empty blocks, rows
without keys; the call adds to the fp32 accumulators it is given."""
import math

import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

# (name, B, Hq, Hkv, nq, nk, causal, qg0, qstep, kg0, kstep)
CASES = [
    ("contig_diagonal_ragged", 1, 2, 2, 300, 300, True, 0, 1, 0, 1),
    ("contig_full_past_block", 1, 2, 2, 256, 192, True, 512, 1, 0, 1),
    ("striped_src_le_rank", 1, 2, 1, 260, 260, True, 2, 4, 1, 4),
    ("striped_src_gt_rank", 1, 2, 2, 260, 260, True, 1, 4, 3, 4),
    ("empty_block", 1, 2, 2, 100, 128, True, 0, 1, 1000, 1),
    ("noncausal_ragged", 2, 2, 2, 130, 520, False, 0, 1, 0, 1),
    ("gqa_4to1", 1, 8, 2, 384, 384, True, 0, 1, 0, 1),
    ("two_tiles_ragged", 1, 2, 2, 100, 100, True, 0, 1, 0, 1),
    ("gqa_8to1_ragged", 1, 8, 1, 130, 130, True, 0, 1, 0, 1),
    ("tiny", 1, 1, 1, 1, 1, True, 0, 1, 0, 1),
    ("no_keys", 1, 2, 2, 70, 0, True, 0, 1, 0, 1),
]


ABS_FLOOR = 2e-6  # fp32 resolution of an accumulator holding values of magnitude ~4


def check_grad(got, ref, what, rel_max=1e-2, rel_mean=2e-3):
    """Gradient bound, relative to the reference's own scale (see the design notes):
    max |err| <= rel_max * max |ref| + ABS_FLOOR and mean |err| <= rel_mean * mean |ref|
    + ABS_FLOOR."""
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), "%s: non-finite" % what
    if not ref.size:
        return 0.0
    scale_max = float(np.abs(ref).max())
    scale_mean = float(np.abs(ref).mean())
    assert err.max() <= rel_max * scale_max + ABS_FLOOR, "%s: max err %.3e vs max|ref| %.3e" % (
        what, err.max(), scale_max)
    assert err.mean() <= rel_mean * scale_mean + ABS_FLOOR, "%s: mean err %.3e vs mean|ref| %.3e" % (
        what, err.mean(), scale_mean)
    return float(err.max() / max(scale_max, 1e-30))


def run_case(case, dtype, d, seed=0):
    import torch
    name, B, Hq, Hkv, nq, nk, causal, qg0, qs, kg0, ks = case
    sd = 300 + seed
    xs = {}
    for nm, shape, s_ in (("q", (B, Hq, nq, d), 1), ("k", (B, Hkv, nk, d), 2),
                          ("v", (B, Hkv, nk, d), 3), ("g", (B, Hq, nq, d), 4)):
        xs[nm] = inputs.to_dtype(inputs.normal(shape, sd + s_), dtype)
    qf, kf, vf, gf = xs["q"][1], xs["k"][1], xs["v"][1], xs["g"][1]
    scale = 1.0 / math.sqrt(d)
    # the "forward" here is this block alone: lse and O of its partial
    ro, rm, rl = oracle.block_partial(qf, kf, vf, scale, causal, qg0, qs, kg0, ks)
    with np.errstate(divide="ignore"):
        lse = np.where(rl > 0, rm + np.log(np.where(rl > 0, rl, 1.0)), -np.inf)
    o_st, o_f = inputs.to_dtype(ro.astype(np.float32), dtype)   # O as the forward hands it over
    Dv = (gf.astype(np.float64) * o_f.astype(np.float64)).sum(-1)
    qid = qg0 + qs * np.arange(nq)
    kid = kg0 + ks * np.arange(nk)
    rq, rk, rv = oracle.block_bwd(qf, kf, vf, gf, lse, Dv, scale, causal, qid, kid)

    dev = lambda st: parity.to_device(st, dtype)
    q, k, v, g, o = dev(xs["q"][0]), dev(xs["k"][0]), dev(xs["v"][0]), dev(xs["g"][0]), dev(o_st)
    lse_d = torch.from_numpy(lse.astype(np.float32)).cuda()
    rng = np.random.default_rng(seed)
    base = {nm: rng.standard_normal(shape).astype(np.float32)
            for nm, shape in (("dq", (B, Hq, nq, d)), ("dk", (B, Hkv, nk, d)),
                              ("dv", (B, Hkv, nk, d)))}
    dq, dk, dv = (torch.from_numpy(base[nm]).cuda() for nm in ("dq", "dk", "dv"))
    a = rb.block_bwd_args(q, k, v, o, g, lse_d, dq, dk, dv, scale, causal, qg0, qs, kg0, ks)
    ws = torch.empty(max(rb.ra_block_bwd_workspace_size(a), 256), dtype=torch.uint8,
                     device="cuda")
    rb.ra_block_bwd(a, ws)
    torch.cuda.synchronize()
    out = {}
    for nm, t, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        got = t.cpu().numpy().astype(np.float64) - base[nm]
        out[nm] = check_grad(got, ref, "%s %s %s d=%d" % (name, nm, dtype, d))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_block_bwd_matches_oracle(case, dtype, d):
    run_case(case, dtype, d)
