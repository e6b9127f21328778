"""ra_decode_fwd (a few new queries against a KV cache split over R ranks)
against the fp64 oracle's attention of the same query tokens over the whole
cache in token order: MHA and grouped heads, d 64 and 128, 1 to 16 new
tokens (one and two 32-column blocks), queries at the end of the cache and in
its middle (later shards fully masked), non-causal, ragged and tiny shards,
an empty cache, and the full-size 1M-token cache."""
import math

import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

# (name, B, Hq, Hkv, d, R, n, nq, q_gid0 (None: the last nq tokens), causal, dtype)
CASES = [
    ("mha_one_token", 1, 4, 4, 128, 4, 1000, 1, None, True, "bf16"),
    ("gqa4_16_tokens_two_col_blocks", 1, 8, 2, 64, 8, 300, 16, None, True, "fp16"),
    ("gqa8_mid_sequence", 2, 8, 1, 128, 2, 4096, 4, 3000, True, "bf16"),
    ("noncausal_ragged", 1, 4, 2, 64, 3, 777, 3, None, False, "bf16"),
    ("tiny_shards", 1, 2, 2, 128, 5, 1, 2, None, True, "fp16"),
    ("query_before_cache_start", 1, 2, 1, 64, 2, 64, 2, 0, True, "bf16"),
    ("many_ranks", 1, 4, 4, 128, 64, 96, 8, None, True, "bf16"),
]


def make(case, seed):
    name, B, Hq, Hkv, d, R, n, nq, q0, causal, dtype = case
    S = R * n
    q32 = inputs.normal((B, Hq, nq, d), seed + 1)
    k32 = inputs.normal((B, Hkv, S, d), seed + 2)
    v32 = inputs.normal((B, Hkv, S, d), seed + 3)
    qs, qf = inputs.to_dtype(q32, dtype)
    ks, kf = inputs.to_dtype(k32, dtype)
    vs, vf = inputs.to_dtype(v32, dtype)
    return (qs, qf), (ks, kf), (vs, vf)


def run_decode(case, q, k, v):
    """q [B][Hq][nq][d], k, v [B][Hkv][S][d] (device, token order) -> (o, lse) on device."""
    import torch
    name, B, Hq, Hkv, d, R, n, nq, q0, causal, dtype = case
    S = R * n
    q0 = S - nq if q0 is None else q0
    # contiguous split: shard r holds tokens r*n .. r*n + n - 1
    k_sh = k.view(B, Hkv, R, n, d).permute(2, 0, 1, 3, 4).contiguous()
    v_sh = v.view(B, Hkv, R, n, d).permute(2, 0, 1, 3, 4).contiguous()
    nbytes = rb.ra_packed_v_bytes(rb.dtype_code(v), R * B, Hkv, n, d)
    vp = torch.empty(max(nbytes // 2, 8), dtype=v.dtype, device="cuda")
    if n > 0:
        rb.ra_pack_v(v_sh.view(R * B, Hkv, n, d), vp)
    o = torch.full((B, Hq, nq, d), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, Hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    a = rb.decode_args(q, k_sh, vp, o, lse, 1 / math.sqrt(d), causal, q0)
    ws = torch.empty(rb.ra_decode_fwd_workspace_size(a), dtype=torch.uint8, device="cuda")
    rb.ra_decode_fwd(a, ws)
    torch.cuda.synchronize()
    return o, lse, q0


def reference(case, qf, kf, vf, q0):
    name, B, Hq, Hkv, d, R, n, nq, _, causal, dtype = case
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(nq), indexing="ij")
    t = (q0 + ii).ravel()
    ro, rl = oracle.attention_rows(qf[bb.ravel(), hh.ravel(), ii.ravel()], bb.ravel(), hh.ravel(),
                                   t, kf, vf, Hq, 1 / math.sqrt(d), causal)
    return ro.reshape(B, Hq, nq, d), rl.reshape(B, Hq, nq)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_decode_matches_oracle(case):
    (qs, qf), (ks, kf), (vs, vf) = make(case, 700)
    dtype = case[-1]
    q, k, v = (parity.to_device(x, dtype) for x in (qs, ks, vs))
    o, lse, q0 = run_decode(case, q, k, v)
    ro, rl = reference(case, qf, kf, vf, q0)
    go, gl = parity.to_f64(o), parity.to_f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), "empty-row pattern"
    assert (go[empty] == 0).all()
    parity.check_o(go, np.where(empty[..., None], 0.0, ro), case[0])
    parity.check_lse(gl, rl, case[0])


def test_decode_empty_cache():
    import torch
    case = ("empty", 1, 4, 2, 64, 3, 0, 2, 0, True, "bf16")
    q = torch.randn(1, 4, 2, 64, device="cuda").to(torch.bfloat16)
    kv = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse, _ = run_decode(case, q, kv, kv)
    assert (o == 0).all() and torch.isneginf(lse).all()


def test_decode_deterministic():
    case = CASES[1]
    (qs, _), (ks, _), (vs, _) = make(case, 701)
    q, k, v = (parity.to_device(x, case[-1]) for x in (qs, ks, vs))
    a = run_decode(case, q, k, v)
    b = run_decode(case, q, k, v)
    import torch
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_full_size_1m_cache():
    """The decode workload at full size: 1,048,576-token cache over 8 ranks, 32 query
    heads on 8 K/V heads, d = 128, 4 new tokens at the end, bf16; every row."""
    from long_context_exact_block_amd import configs
    w = configs.DECODE_1M
    case = ("decode_1M", w.B, w.Hq, w.Hkv, w.d, w.R, w.n, w.nq, None, True, w.dtype)
    (qs, qf), (ks, kf), (vs, vf) = make(case, w.seed)
    q, k, v = (parity.to_device(x, w.dtype) for x in (qs, ks, vs))
    o, lse, q0 = run_decode(case, q, k, v)
    ro, rl = reference(case, qf, kf, vf, q0)
    parity.check_o(parity.to_f64(o), ro, "decode_1M")
    parity.check_lse(parity.to_f64(lse), rl, "decode_1M")
