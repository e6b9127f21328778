"""The identities the full-size backward test checks over every key
(parity.bwd_sum_errors, parity.bwd_identity_errors), on the CPU: the fp64
oracle's exact gradients satisfy them to rounding, gradients rounded to 16 bits
stay well within the test's bound, and planted mistakes of the kinds a kernel
could make exceed it in at least one of them.  The inner-product identities are
blind to a dropped key tile (a third of the keys moves them by under 5 % of
their norm); the sums catch it."""
import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import inputs
from tests import parity

B, HQ, HKV, S, D = 1, 4, 2, 192, 64
SCALE = D ** -0.5


@pytest.fixture(scope="module")
def case():
    import torch
    data = inputs.qkv(B, HQ, HKV, S, D, 77, "bf16")
    q, k, v = data["q32"], data["k32"], data["v32"]
    dout = inputs.to_dtype(inputs.normal((B, HQ, S, D), 78), "bf16")[1]
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, SCALE, True)
    o, _ = oracle.attention_full(q, k, v, SCALE, True)
    t = {n: torch.from_numpy(np.ascontiguousarray(x)) for n, x in
         (("dq", dq), ("dk", dk), ("dv", dv), ("o", o))}
    return t, (q, k, v, dout)


def errors(t, host, **planted):
    """The four identities' largest errors: dq/dk and dv/O inner products, dv and dk sums."""
    g = dict(t, **planted)
    rows = np.ones(S, bool)
    ip = parity.bwd_identity_errors(g["dq"], g["dk"], g["dv"], g["o"], *host, HQ // HKV)
    sm = parity.bwd_sum_errors(g["dk"], g["dv"], host[3], rows, HQ // HKV)
    return np.concatenate([ip.max(axis=(0, 1)), sm.max(axis=(0, 1))])


def test_exact_gradients_satisfy_the_identities(case):
    t, host = case
    assert errors(t, host).max() < 1e-12


def test_rounded_gradients_stay_within_the_bound(case):
    import torch
    t, host = case
    rounded = {n: x.to(torch.bfloat16).double() for n, x in t.items()}
    e = errors(rounded, host)
    assert e.max() <= parity.BWD_SUM_REL / 5, e


def test_planted_mistakes_exceed_the_bound(case):
    import torch
    t, host = case
    q, k, v, dout = host
    dk_tile = t["dk"].clone()
    dk_tile[:, :, 64:128] = 0                              # one 64-key tile of dk dropped
    dk_swap = t["dk"].flip(1)                              # K/V heads swapped
    dv_shift = torch.roll(t["dv"], 1, dims=2)              # dv of key j stored at j + 1
    dq_nc, dk_nc, _ = oracle.attention_bwd(q, k, v, dout, SCALE, False)  # mask missing
    o_nc, _ = oracle.attention_full(q, k, v, SCALE, False)
    dv_tile = t["dv"].clone()
    dv_tile[:, :, 128:192] = 0                             # one 64-key tile of dv dropped
    plants = {
        "dk tile dropped": dict(dk=dk_tile),
        "dv tile dropped": dict(dv=dv_tile),
        "dq scale halved": dict(dq=t["dq"] * 0.5),
        "dk unmasked": dict(dk=torch.from_numpy(dk_nc)),
        "dk heads swapped": dict(dk=dk_swap),
        "dv off by one key": dict(dv=dv_shift),
        "O unmasked": dict(o=torch.from_numpy(o_nc)),
    }
    for name, planted in plants.items():
        e = errors(t, host, **planted)
        assert e.max() > parity.BWD_SUM_REL, "%s not caught (%s)" % (name, e)
