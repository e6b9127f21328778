"""The five workloads at full size, in the launch configuration the benchmark
times (FORWARD hand-off: on the 512-token shards the block kernel writes each
block on to the next rank, elsewhere the side copy as in COPY; fused
online-softmax fold; original-order pipeline), compared with the fp64 oracle on
seeded samples of query rows computed one by one over their full allowed key
sets.  Where the block kernel forwards, the COPY hand-off's outputs at full size
must be bitwise equal.  The sample always contains token 0 and
token S-1 when owned, and the first and last local row of every computed rank
(under the striped layout the first local row is the row that sees no key in
blocks coming from higher ranks)."""
import gc

import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import configs, inputs
from long_context_exact_block_amd.pipeline import RingAttention
from tests import parity

pytestmark = pytest.mark.gpu

RANDOM_ROWS = {1: 2048, 2: 192, 3: 4096, 4: 4096, 5: 4096}


def forwards_in_kernel(w, layout):
    """Whether the FORWARD hand-off has the block kernel write blocks on for this
    workload: 16-bit inputs (the packed path), more than one rank, and hops too
    short for the thin side copy to hide (the library's own rule)."""
    if w.dtype == "fp32" or w.R == 1:
        return False
    elt = 2
    kb = w.ranks * w.B * w.Hkv * w.n * w.d * elt
    vb = w.ranks * w.B * w.Hkv * w.d * ((w.n + 63) // 64 * 64) * elt
    pairs = w.ranks * w.B * w.Hq * float(w.n) * w.n * (0.5 if w.causal else 1.0)
    return not rb.thin_handoff(2.0 * (kb + vb), pairs, w.d)


def _cases():
    for w in configs.ALL:
        if w is configs.MHA_32K:  # compared on every row below
            continue
        for layout in w.layouts:
            yield pytest.param(w, layout, id="%s-%s" % (w.name, layout))
    # the 2R-chunk zig-zag layout on the 1M-token share (rank 3 holds chunks 3 and 12)
    yield pytest.param(configs.SHARE_1M, "zigzag", id="%s-zigzag" % configs.SHARE_1M.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,layout", list(_cases()))
def test_full_size_workload(w, layout):
    import torch
    print("\n[full] %s %s: inputs" % (w.name, layout), flush=True)
    data = inputs.qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.seed, w.dtype, w.q_scale)
    tdt = parity.torch_dtype(w.dtype)
    q = parity.to_device(data["q"], w.dtype)
    k = parity.to_device(data["k"], w.dtype)
    v = parity.to_device(data["v"], w.dtype)
    for key in ("q", "k", "v"):
        del data[key]
    o = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
    lse = torch.full((w.B, w.Hq, w.S), float("nan"), dtype=torch.float32, device="cuda")
    ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                       rank0=w.rank0, n_ranks=w.ranks, handoff=rb.HANDOFF_FORWARD)
    print("[full] %s %s: ring" % (w.name, layout), flush=True)
    ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()
    if forwards_in_kernel(w, layout):
        print("[full] %s %s: ring with the COPY hand-off" % (w.name, layout), flush=True)
        o2 = torch.zeros_like(o)
        lse2 = torch.full_like(lse, float("nan"))
        RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                      rank0=w.rank0, n_ranks=w.ranks, handoff=rb.HANDOFF_COPY).run(
                          q, k, v, o2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(o, o2), "%s %s: FORWARD and COPY outputs differ" % (w.name, layout)
        assert torch.equal(lse, lse2), "%s %s: FORWARD and COPY LSE differ" % (w.name, layout)
        del o2, lse2

    fwd, _ = oracle.layout_maps(rb.LAYOUTS[layout], w.S, w.R)
    special, picks = parity.sample_tokens(fwd, w.n, w.rank0, w.ranks, RANDOM_ROWS[w.index],
                                          seed=w.seed + 7)
    rng = np.random.default_rng(w.seed + 8)
    rows_b, rows_h, rows_t = [], [], []
    for t in special:
        for b in sorted({0, w.B - 1}):
            for h in sorted({0, w.Hq // 2, w.Hq - 1}):
                rows_b.append(b), rows_h.append(h), rows_t.append(t)
    rows_b += list(rng.integers(0, w.B, len(picks)))
    rows_h += list(rng.integers(0, w.Hq, len(picks)))
    rows_t += list(picks)
    rb_, rh_, rt_ = (np.asarray(x, np.int64) for x in (rows_b, rows_h, rows_t))
    print("[full] %s %s: oracle on %d rows" % (w.name, layout, len(rt_)), flush=True)
    q32 = data["q32"]
    ro, rl = oracle.attention_rows(q32[rb_, rh_, rt_], rb_, rh_, rt_, data["k32"], data["v32"],
                                   w.Hq, w.scale, w.causal)
    idx = (torch.from_numpy(rb_), torch.from_numpy(rh_), torch.from_numpy(rt_))
    go = o.cpu()[idx].double().numpy()
    gl = lse.cpu()[idx].double().numpy()
    mx, mean = parity.check_o(go, ro, w.name)
    lmx = parity.check_lse(gl, rl, w.name)
    print("[full] %s %s: O max %.3e mean %.3e LSE max %.3e" % (w.name, layout, mx, mean, lmx),
          flush=True)
    del data, q32, q, k, v, o, lse, ra
    gc.collect()
    torch.cuda.empty_cache()


_MHA_OUT = {}


def _mha_32k_outputs():
    """Both layouts' outputs of the 32k MHA workload (computed once, kept on the host)."""
    import torch
    if _MHA_OUT:
        return _MHA_OUT
    w = configs.MHA_32K
    data = inputs.qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.seed, w.dtype, w.q_scale)
    tdt = parity.torch_dtype(w.dtype)
    q = parity.to_device(data["q"], w.dtype)
    k = parity.to_device(data["k"], w.dtype)
    v = parity.to_device(data["v"], w.dtype)
    for layout in w.layouts:
        o = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
        lse = torch.full((w.B, w.Hq, w.S), float("nan"), dtype=torch.float32, device="cuda")
        ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                           rank0=w.rank0, n_ranks=w.ranks, handoff=rb.HANDOFF_FORWARD)
        ra.run(q, k, v, o, lse)
        torch.cuda.synchronize()
        _MHA_OUT[layout] = (o.cpu().double().numpy(), lse.cpu().double().numpy())
        del ra, o, lse
    del q, k, v
    torch.cuda.empty_cache()
    _MHA_OUT["data"] = data
    return _MHA_OUT


@pytest.mark.timeout(600)
@pytest.mark.parametrize("heads", [(0, 8), (8, 16), (16, 24), (24, 32)],
                         ids=lambda h: "heads%d-%d" % h)
def test_32k_mha_every_row_both_layouts(heads):
    """The 32k MHA workload compared on every query row, for the contiguous and
    the striped layout, against the fp64 oracle over the whole sequence in the
    original token order (1.7e10 allowed pairs in all; a quarter of the heads
    per test)."""
    w = configs.MHA_32K
    h0, h1 = heads
    print("\n[full] %s heads %d-%d: rings" % (w.name, h0, h1), flush=True)
    out = _mha_32k_outputs()
    data = out["data"]
    print("[full] %s heads %d-%d: oracle on every row" % (w.name, h0, h1), flush=True)
    ro, rl = oracle.attention_full(np.ascontiguousarray(data["q32"][:, h0:h1]),
                                   np.ascontiguousarray(data["k32"][:, h0:h1]),
                                   np.ascontiguousarray(data["v32"][:, h0:h1]), w.scale, w.causal)
    for layout in w.layouts:
        o, lse = out[layout]
        err = np.abs(o[:, h0:h1] - ro)
        mx, mean = float(err.max()), float(err.mean())
        assert np.isfinite(err).all() and mx <= parity.O_MAX_ABS and mean <= parity.O_MEAN_ABS, (
            layout, mx, mean)
        lmx = parity.check_lse(lse[:, h0:h1], rl, w.name + " " + layout)
        print("[full] %s %s heads %d-%d every row: O max %.3e mean %.3e LSE max %.3e" % (
            w.name, layout, h0, h1, mx, mean, lmx), flush=True)
    if h1 == w.Hq:
        _MHA_OUT.clear()
