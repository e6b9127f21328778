"""ra_layout_permute / gather / scatter (bit-exact against the oracle's maps)
and ra_merge / ra_finalize against the fp64 oracle combine."""
import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,R", [(1024, 4), (32768, 8), (131072, 8), (1048576, 8), (32768, 64),
                                 (12, 4), (7, 7), (5, 1), (0, 3), (16, 4), (2, 1)])
@pytest.mark.parametrize("layout", [rb.LAYOUT_CONTIGUOUS, rb.LAYOUT_STRIPED, rb.LAYOUT_ZIGZAG])
def test_permute_bit_exact(S, R, layout):
    import torch
    if layout == rb.LAYOUT_ZIGZAG and S % (2 * R):
        pytest.skip("zig-zag needs S % 2R == 0 (rejected, see test_abi)")
    fwd = torch.full((max(S, 1),), -1, dtype=torch.int32, device="cuda")
    inv = torch.full((max(S, 1),), -1, dtype=torch.int32, device="cuda")
    rb.ra_layout_permute(layout, S, R, fwd, inv)
    torch.cuda.synchronize()
    if S == 0:
        return
    of, oi = oracle.layout_maps(layout, S, R)
    assert np.array_equal(fwd.cpu().numpy(), of)
    assert np.array_equal(inv.cpu().numpy(), oi)


@pytest.mark.parametrize("dtype,d", [("int16", 128), ("int16", 64), ("float32", 64),
                                     ("float32", 1), ("int8", 3)])
@pytest.mark.parametrize("rank0,n_ranks", [(0, 4), (3, 1), (1, 2)])
def test_gather_scatter_bit_exact(dtype, d, rank0, n_ranks):
    import torch
    B, H, S, R = 2, 3, 64, 4
    n = S // R
    rng = np.random.default_rng(5)
    x = rng.integers(-1000, 1000, (B, H, S, d)).astype(dtype)
    for layout in (rb.LAYOUT_CONTIGUOUS, rb.LAYOUT_STRIPED, rb.LAYOUT_ZIGZAG):
        of, _ = oracle.layout_maps(layout, S, R)
        fwd = torch.from_numpy(of).cuda()
        xd = torch.from_numpy(x).cuda()
        xs = torch.zeros((n_ranks, B, H, n, d), dtype=xd.dtype, device="cuda")
        rb.ra_layout_gather(xd, xs, fwd, R, rank0, n_ranks)
        expect = np.stack([x[:, :, of[(rank0 + k) * n:(rank0 + k + 1) * n]]
                           for k in range(n_ranks)])
        assert np.array_equal(xs.cpu().numpy(), expect)
        back = torch.full_like(xd, 7)
        rb.ra_layout_scatter(xs, back, fwd, R, rank0, n_ranks)
        b = back.cpu().numpy()
        owned = of[rank0 * n:(rank0 + n_ranks) * n]
        mask = np.zeros(S, bool)
        mask[owned] = True
        assert np.array_equal(b[:, :, mask], x[:, :, mask])
        assert (b[:, :, ~mask] == 7).all()


def test_gather_scatter_many_slabs():
    """More (rank, batch, head) slabs than a 2-D grid's y extent: the 1-D kernel."""
    import torch
    B, H, S, R, d = 1, 70000, 4, 4, 8  # 16-byte rows, 4 * 70000 shard slabs
    n = S // R
    x = torch.arange(B * H * S * d, dtype=torch.int32).remainder(30011).to(torch.int16)
    x = x.view(B, H, S, d)
    of, _ = oracle.layout_maps(rb.LAYOUT_STRIPED, S, R)
    fwd = torch.from_numpy(of).cuda()
    xd = x.cuda()
    xs = torch.zeros((R, B, H, n, d), dtype=torch.int16, device="cuda")
    rb.ra_layout_gather(xd, xs, fwd, R, 0, R)
    xn = x.numpy()
    expect = np.stack([xn[:, :, of[k * n:(k + 1) * n]] for k in range(R)])
    assert np.array_equal(xs.cpu().numpy(), expect)
    back = torch.zeros_like(xd)
    rb.ra_layout_scatter(xs, back, fwd, R, 0, R)
    assert torch.equal(back.cpu(), x)


def _partials(rows, d, seed, empty_frac=0.1):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, d)).astype(np.float32)
    m = (3 * rng.standard_normal(rows)).astype(np.float32)
    l = np.exp(rng.standard_normal(rows)).astype(np.float32) + 0.5
    e = rng.random(rows) < empty_frac
    o[e] = 0
    m[e] = -np.inf
    l[e] = 0
    return o, m, l


@pytest.mark.parametrize("rows,d", [(1, 64), (1000, 64), (777, 128), (4096, 128)])
def test_merge_matches_oracle(rows, d):
    import torch
    a = _partials(rows, d, 1)
    b = _partials(rows, d, 2)
    b[1][:5] = -np.inf  # some rows empty on one side only
    b[2][:5] = 0
    b[0][:5] = 0
    ro, rm, rl = oracle.merge(*a, *b)
    ta = [torch.from_numpy(x.copy()).cuda() for x in a]
    tb = [torch.from_numpy(x.copy()).cuda() for x in b]
    rb.ra_merge(*ta, *tb)
    torch.cuda.synchronize()
    go, gm, gl = (t.cpu().numpy().astype(np.float64) for t in ta)
    assert np.array_equal(np.isneginf(gm), np.isneginf(rm))
    fin = ~np.isneginf(rm)
    assert np.abs(gm[fin] - rm[fin]).max(initial=0) == 0  # max is exact
    assert np.allclose(gl, rl, rtol=1e-5, atol=0)
    assert np.allclose(go, ro, rtol=0, atol=1e-5)
    assert (go[~fin] == 0).all() and (gl[~fin] == 0).all()


# (rows, d, output offset in elements): d % 8 == 0 with a 16-byte aligned output
# takes the 8-wide kernel, the others the 4-wide one
@pytest.mark.parametrize("rows,d,off", [(513, 128, 0), (77, 64, 0), (300, 12, 0), (129, 128, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_finalize(dtype, rows, d, off):
    import torch
    o, m, l = _partials(rows, d, 3)
    buf = torch.empty(rows * d + off, dtype=parity.torch_dtype(dtype), device="cuda")
    out = buf[off:].view(rows, d)
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    rb.ra_finalize(torch.from_numpy(o).cuda(), torch.from_numpy(m).cuda(),
                   torch.from_numpy(l).cuda(), out, lse)
    torch.cuda.synchronize()
    ref = torch.from_numpy(o).to(parity.torch_dtype(dtype))  # CPU round-to-nearest-even
    assert torch.equal(out.cpu(), ref)
    expect = np.where(l > 0, m.astype(np.float64) + np.log(np.where(l > 0, l, 1)), -np.inf)
    parity.check_lse(lse.cpu().numpy(), expect, "finalize")


@pytest.mark.parametrize("thin", [False, True])
@pytest.mark.parametrize("nbytes,dst_off,src_off", [
    (16, 0, 0), (4096, 0, 0), (256 * 64 * 16 * 4 + 48, 0, 0), (536870912 // 64, 0, 0),
    (1024 * 1024 * 3 + 1024 * 5 + 16 * 7, 0, 0), (1000, 0, 0), (4096, 2, 0), (4096, 0, 6),
    (37, 1, 3), (0, 0, 0)])
def test_handoff_copy_bit_exact(nbytes, dst_off, src_off, thin):
    """ra_handoff_copy moves exactly `nbytes` bytes in both forms: 16-byte aligned
    copies take the kernels (sizes below, at and past the grids' strides and
    unrolls, runs of an odd number of 1 KB units per workgroup, workgroups past
    the data, and ragged tails), the rest the runtime copy; bytes around the
    destination stay."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes + 7 * dst_off + src_off)
    src = torch.randint(0, 256, (nbytes + src_off + 32,), dtype=torch.uint8, device="cuda",
                        generator=g)
    dst = torch.full((nbytes + dst_off + 32,), 0xA5, dtype=torch.uint8, device="cuda")
    before = dst.clone()
    rb.ra_handoff_copy(dst[dst_off:], src[src_off:], nbytes, thin=thin)
    torch.cuda.synchronize()
    got, ref = dst.cpu().numpy(), before.cpu().numpy()
    ref[dst_off:dst_off + nbytes] = src.cpu().numpy()[src_off:src_off + nbytes]
    assert np.array_equal(got, ref)

