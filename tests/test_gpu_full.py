"""The five workloads at full size, in the launch configuration the benchmark
times (COPY hand-off, fused online-softmax fold, original-order pipeline),
compared with the fp64 oracle on seeded samples of query rows computed one by
one over their full allowed key sets.  The sample always contains token 0 and
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

RANDOM_ROWS = {1: 256, 2: 192, 3: 128, 4: 48, 5: 256}


def _cases():
    for w in configs.ALL:
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
                       rank0=w.rank0, n_ranks=w.ranks)
    print("[full] %s %s: ring" % (w.name, layout), flush=True)
    ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()

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
