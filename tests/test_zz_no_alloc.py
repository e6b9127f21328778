"""ra_decode_fwd_noalloc, the decode entry point for callers that cannot
allocate (partials in the library's per-GPU device array), against
ra_decode_fwd with a caller workspace: the same kernels on the same inputs,
so the outputs must be bitwise equal.  Two calls in a row, the second with a
smaller input (the array keeps the first call's partials), then the first
shape again."""
import ctypes
import math

import pytest

from long_context_exact_block_amd import binding as rb

pytestmark = pytest.mark.gpu

# (name, B, Hq, Hkv, d, R, n, nq, causal, dtype)
BIG = ("gqa4_1M_cache_4_tokens", 1, 32, 8, 128, 8, 131072, 4, True, "bf16")
SMALL = ("mha_ragged_noncausal", 1, 4, 4, 64, 3, 777, 2, False, "fp16")


def make(case, seed):
    import torch
    name, B, Hq, Hkv, d, R, n, nq, causal, dtype = case
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((B, Hq, nq, d), device="cuda", generator=g).to(td)
    k_sh = torch.randn((R, B, Hkv, n, d), device="cuda", generator=g).to(td)
    v_sh = torch.randn((R, B, Hkv, n, d), device="cuda", generator=g).to(td)
    nbytes = rb.ra_packed_v_bytes(rb.dtype_code(v_sh), R * B, Hkv, n, d)
    vp = torch.empty(nbytes // 2, dtype=td, device="cuda")
    rb.ra_pack_v(v_sh.view(R * B, Hkv, n, d), vp)
    return q, k_sh, vp


def decode(case, tensors, noalloc):
    import torch
    name, B, Hq, Hkv, d, R, n, nq, causal, dtype = case
    q, k_sh, vp = tensors
    o = torch.full((B, Hq, nq, d), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, Hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    a = rb.decode_args(q, k_sh, vp, o, lse, 1 / math.sqrt(d), causal, R * n - nq)
    if noalloc:
        rb.ra_decode_fwd_noalloc(a)
    else:
        ws = torch.empty(rb.ra_decode_fwd_workspace_size(a), dtype=torch.uint8, device="cuda")
        rb.ra_decode_fwd(a, ws)
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_equals_workspace_on_two_calls_in_a_row():
    import torch
    print("noalloc decode: %s then %s then %s" % (BIG[0], SMALL[0], BIG[0]), flush=True)
    data = {c[0]: make(c, 90 + i) for i, c in enumerate((BIG, SMALL))}
    for case in (BIG, SMALL, BIG):
        got = decode(case, data[case[0]], noalloc=True)
        ref = decode(case, data[case[0]], noalloc=False)
        for x, y in zip(got, ref):
            assert bool(torch.isfinite(x.float()).all()), case[0]
            assert torch.equal(x, y), case[0]


def test_noalloc_rejects_partials_beyond_its_array():
    lib = rb.lib()
    a = rb.DecodeArgs()
    a.q = a.k = a.v = a.o = a.lse = 4096
    a.dtype, a.R, a.B, a.Hq, a.Hkv, a.nq, a.n, a.d = rb.DT_BF16, 2, 64, 64, 64, 16, 128, 128
    a.scale, a.causal, a.q_gid0 = 0.088, 1, 0
    assert lib.ra_decode_fwd_workspace_size(ctypes.byref(a)) > 32 << 20
    assert lib.ra_decode_fwd_noalloc(ctypes.byref(a), None) == 6
    assert "32" in rb.last_error()
