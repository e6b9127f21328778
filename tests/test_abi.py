"""The C ABI library: builds, loads, exports what include/ra.h declares, and
rejects bad arguments on the host before touching the GPU (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import build as rbuild
from tests import oracle_pins as pins

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "ra.h")


@pytest.fixture(scope="module")
def lib():
    rbuild.build(force=False)
    return rb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("ra_layout_permute", "ra_block_fwd", "ra_merge", "ra_ring_fwd",
              "ra_ring_fwd_workspace_size", "ra_status_string", "ra_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(rb.EXPORTED) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.ra_version() >= 100
    for code, name in rb.STATUS_NAMES.items():
        assert lib.ra_status_string(code).decode() == name


def _block(**kw):
    a = rb.BlockArgs()
    a.q = a.k = a.v = a.o = a.m = a.l = 4096
    a.dtype, a.B, a.Hq, a.Hkv, a.n_q, a.n_k, a.d = rb.DT_BF16, 1, 4, 2, 8, 8, 128
    for i, s in enumerate((4 * 8 * 128, 8 * 128, 128)):
        a.q_stride[i] = a.o_stride[i] = s
    for i, s in enumerate((2 * 8 * 128, 8 * 128, 128)):
        a.k_stride[i] = a.v_stride[i] = s
    a.scale, a.causal = 0.088, 1
    a.q_gid0, a.q_gid_step, a.k_gid0, a.k_gid_step = 0, 1, 0, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 9, 3), ("d", 96, 2), ("Hkv", 3, 2), ("Hq", 0, 2), ("n_q", -1, 2),
    ("q_gid_step", 0, 1), ("scale", -1.0, 1), ("scale", float("nan"), 1), ("q", 0, 1),
    ("k", 4097, 4), ("o", 4100, 4), ("v_packed", 2, 1),
])
def test_block_fwd_rejects(lib, field, value, status):
    a = _block(**{field: value})
    st = lib.ra_block_fwd(ctypes.byref(a), None)
    assert st == status, (st, rb.last_error())
    assert rb.last_error()


def test_block_fwd_packed_v_rules(lib):
    a = _block(v_packed=1, dtype=rb.DT_FP32)
    assert lib.ra_block_fwd(ctypes.byref(a), None) == 6  # unsupported for fp32
    a = _block(v_packed=1)
    a.v_stride[2] = 3  # ignored for packed V
    a.q = 0
    assert lib.ra_block_fwd(ctypes.byref(a), None) == 1  # fails on q, not on v_stride


def test_block_fwd_packed_v_size_limits(lib):
    # packed V addresses a (b, h) slice with 32-bit offsets: 2^23 keys, 2^22-element K rows
    a = _block(v_packed=1, n_k=(1 << 23) + 1)
    assert lib.ra_block_fwd(ctypes.byref(a), None) == 6
    a = _block(v_packed=1)
    a.k_stride[2] = (1 << 22) + 128
    assert lib.ra_block_fwd(ctypes.byref(a), None) == 6
    assert "packed V" in rb.last_error()


def test_ring_block_length_limit(lib):
    a = _ring(n=(1 << 23) + 64)
    st = lib.ra_ring_fwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None, None)
    assert st == 6, (st, rb.last_error())


def test_pack_v_sizes_and_rejects(lib):
    assert lib.ra_packed_v_bytes(rb.DT_BF16, 2, 3, 100, 128) == 2 * 3 * 128 * 128 * 2
    assert lib.ra_packed_v_bytes(rb.DT_FP16, 1, 1, 64, 64) == 64 * 64 * 2
    assert lib.ra_packed_v_bytes(rb.DT_FP32, 1, 1, 64, 64) == 0
    st = (rb.I64 * 3)(8 * 128, 128, 128)
    assert lib.ra_pack_v(4096, 8192, rb.DT_FP32, 1, 1, 8, 128, st, None) == 3
    assert lib.ra_pack_v(4096, 8192, rb.DT_BF16, 1, 1, 8, 96, st, None) == 2
    assert lib.ra_pack_v(4098, 8192, rb.DT_BF16, 1, 1, 8, 128, st, None) == 4
    assert lib.ra_pack_v(None, 8192, rb.DT_BF16, 1, 1, 8, 128, st, None) == 1


def test_block_fwd_rejects_bad_stride(lib):
    a = _block()
    a.q_stride[2] = 100  # rows no longer 16-byte aligned
    assert lib.ra_block_fwd(ctypes.byref(a), None) == 4


def _ring(**kw):
    a = rb.RingArgs()
    a.q_sh = a.k_sh = a.v_sh = a.o = a.lse = 4096
    a.dtype, a.R, a.rank0, a.n_ranks = rb.DT_BF16, 8, 0, 8
    a.B, a.Hq, a.Hkv, a.n, a.d = 1, 4, 2, 256, 128
    a.scale, a.causal, a.layout, a.handoff, a.merge_mode = 0.088, 1, 1, 0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("R", 0, 2), ("n_ranks", 9, 2), ("rank0", 8, 2), ("rank0", -1, 2), ("rank0", 1, 2), ("layout", 5, 1),
    ("handoff", 3, 1), ("merge_mode", 7, 1), ("dtype", -1, 3), ("d", 32, 2), ("Hkv", 3, 2),
    ("q_sh", 0, 1), ("o", 4104, 4),
])
def test_ring_rejects(lib, field, value, status):
    a = _ring(**{field: value})
    st = lib.ra_ring_fwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None, None)
    assert st == status, (st, rb.last_error())
    assert lib.ra_ring_fwd_workspace_size(ctypes.byref(a)) == 0


def test_ring_workspace_checks(lib):
    a = _ring()
    need = lib.ra_ring_fwd_workspace_size(ctypes.byref(a))
    elt, blk = 2, 1 * 2 * 256 * 128
    rows = 8 * 1 * 4 * 256
    assert need >= 4 * 8 * blk * elt + rows * 128 * 4 + 2 * rows * 4
    assert lib.ra_ring_fwd(ctypes.byref(a), None, need, None, None) == 5
    assert lib.ra_ring_fwd(ctypes.byref(a), ctypes.c_void_p(4096), need - 1, None, None) == 5
    assert lib.ra_ring_fwd(ctypes.byref(a), ctypes.c_void_p(4096 + 16), need, None, None) == 4
    swap = _ring(handoff=1)
    assert lib.ra_ring_fwd_workspace_size(ctypes.byref(swap)) < need
    forward = _ring(handoff=2)  # the same receive buffers as COPY
    assert lib.ra_ring_fwd_workspace_size(ctypes.byref(forward)) == need
    sep = _ring(merge_mode=1)
    assert lib.ra_ring_fwd_workspace_size(ctypes.byref(sep)) > need


def test_layout_rejects(lib):
    assert lib.ra_layout_permute(0, 10, 4, ctypes.c_void_p(4096), None, None) == 2
    assert lib.ra_layout_permute(2, 12, 4, ctypes.c_void_p(4096), None, None) == 2  # S % 2R
    assert lib.ra_layout_permute(3, 8, 4, ctypes.c_void_p(4096), None, None) == 1
    assert lib.ra_layout_permute(1, 8, 4, None, None, None) == 1
    assert lib.ra_layout_gather(4096, 8192, 4096, 3, 1, 1, 8, 4, 4, 0, 4, None) == 1
    assert lib.ra_layout_gather(4096, 8192, 4096, 2, 1, 1, 8, 4, 4, 2, 3, None) == 2


def test_handoff_copy_rejects(lib):
    for thin in (0, 1):
        assert lib.ra_handoff_copy(None, 4096, 16, thin, None) == 1
        assert lib.ra_handoff_copy(4096, None, 16, thin, None) == 1
        assert lib.ra_handoff_copy(None, None, 0, thin, None) == 0  # nothing to copy: no GPU call
    assert lib.ra_handoff_copy(4096, 4096, 16, 2, None) == 1


def test_handoff_form_rule(lib):
    """The copy form the rings pick (ra_handoff_thin): the thin copy beside long hops
    (the 1M-token share, 4096-token blocks, the backward on the 1M share), the
    64-workgroup copy for 512-token shards and tiny rings."""
    def form(B, Hq, Hkv, n, d, ranks, causal, elt=2, work=1.0):
        moved = 2.0 * ranks * 2 * B * Hkv * n * d * elt
        pairs = ranks * B * Hq * float(n) * n * (0.5 if causal else 1.0)
        return rb.thin_handoff(moved, pairs, d, work)
    assert form(1, 8, 8, 131072, 128, 1, True)                   # 1M share, rank 3 of 8
    assert form(1, 8, 8, 131072, 128, 1, True, work=3.2)         # its backward
    assert form(1, 32, 32, 4096, 128, 8, True)                   # 32k MHA, R = 8
    assert form(1, 32, 8, 16384, 128, 8, True)                   # 128k GQA, R = 8
    assert not form(4, 16, 16, 512, 64, 64, False)               # 512-token shards, R = 64
    assert not form(1, 2, 2, 256, 64, 4, True, elt=4)            # tiny fp32 ring
    assert lib.ra_handoff_thin(0.0, 0.0, 128, 1.0) == 0          # nothing to hide behind


def test_merge_finalize_reject(lib):
    assert lib.ra_merge(4096, 4096, 4096, 4096, 4096, 4096, 10, 6, None) == 2
    assert lib.ra_merge(4100, 4096, 4096, 4096, 4096, 4096, 10, 8, None) == 4
    assert lib.ra_merge(None, 4096, 4096, 4096, 4096, 4096, 10, 8, None) == 1
    assert lib.ra_finalize(4096, 4096, 4096, 4096, 4096, 5, 10, 8, None) == 3


@pytest.mark.parametrize("S,R", [(8, 2), (16, 4), (24, 4), (32, 8), (64, 8), (60, 6), (48, 3),
                                 (128, 16), (1024, 4), (512, 64)])
def test_causal_work_matches_oracle_brute_force(lib, ora, S, R):
    """The library's per-rank causal work equals brute-force counting (bit-exact)."""
    for layout in pins.layouts_for(S, R):
        assert np.array_equal(rb.ra_causal_work(layout, S, R), ora.pair_counts(layout, S, R))


@pytest.mark.parametrize("S,R", [(32768, 8), (131072, 8), (1048576, 8), (32768, 64)])
def test_causal_work_closed_forms_at_full_size(lib, S, R):
    for layout in (rb.LAYOUT_CONTIGUOUS, rb.LAYOUT_STRIPED, rb.LAYOUT_ZIGZAG):
        W = rb.ra_causal_work(layout, S, R)
        assert np.array_equal(W, pins.closed_form_counts(layout, S, R))
        assert W.sum() == S * (S + 1) // 2
    # zig-zag: every rank the same causal work
    assert len(set(rb.ra_causal_work(rb.LAYOUT_ZIGZAG, S, R).tolist())) == 1


def test_ring_rejects_odd_zigzag_blocks(lib):
    a = _ring(layout=2, n=255)
    st = lib.ra_ring_fwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None, None)
    assert st == 2 and "even" in rb.last_error()


def _decode(**kw):
    a = rb.DecodeArgs()
    a.q = a.k = a.v = a.o = a.lse = 4096
    a.dtype, a.R, a.B, a.Hq, a.Hkv, a.nq, a.n, a.d = rb.DT_BF16, 8, 1, 32, 8, 4, 131072, 128
    a.scale, a.causal, a.q_gid0 = 0.088, 1, 8 * 131072 - 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("dtype", rb.DT_FP32, 6), ("dtype", 7, 3), ("d", 96, 2), ("Hkv", 5, 2), ("nq", 0, 2),
    ("nq", 65, 2), ("R", 0, 2), ("n", -1, 2), ("n", (1 << 23) + 1, 6), ("scale", 0.0, 1),
    ("q", 0, 1), ("k", 4100, 4),
])
def test_decode_rejects(lib, field, value, status):
    a = _decode(**{field: value})
    st = lib.ra_decode_fwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None)
    assert st == status, (st, rb.last_error())
    assert lib.ra_decode_fwd_workspace_size(ctypes.byref(a)) == 0


def test_decode_workspace(lib):
    a = _decode()
    need = lib.ra_decode_fwd_workspace_size(ctypes.byref(a))
    rows = 1 * 32 * 4
    assert need >= 8 * rows * (128 + 2) * 4  # at least one partial (O, m, l) per rank and row
    assert lib.ra_decode_fwd(ctypes.byref(a), ctypes.c_void_p(4096), need - 1, None) == 5
    assert lib.ra_decode_fwd(ctypes.byref(a), ctypes.c_void_p(4096 + 16), need, None) == 5


def _block_bwd(**kw):
    a = rb.BlockBwdArgs()
    for f in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"):
        setattr(a, f, 4096)
    a.dtype, a.B, a.Hq, a.Hkv, a.n_q, a.n_k, a.d = rb.DT_BF16, 1, 4, 2, 300, 200, 128
    a.scale, a.causal = 0.088, 1
    a.q_gid0, a.q_gid_step, a.k_gid0, a.k_gid_step = 0, 1, 0, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("dtype", rb.DT_FP32, 6), ("dtype", 9, 3), ("d", 96, 2), ("Hkv", 3, 2), ("B", 0, 2),
    ("n_q", -1, 2), ("n_k", (1 << 23) + 1, 6), ("q_gid_step", 0, 1), ("scale", 0.0, 1),
    ("dout", 0, 1), ("lse", 0, 1), ("dk", 0, 1), ("dq", 4100, 4), ("v", 4104, 4),
])
def test_block_bwd_rejects(lib, field, value, status):
    a = _block_bwd(**{field: value})
    st = lib.ra_block_bwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None)
    assert st == status, (st, rb.last_error())
    assert lib.ra_block_bwd_workspace_size(ctypes.byref(a)) == 0


def test_block_bwd_workspace_and_empty(lib):
    a = _block_bwd()
    need = lib.ra_block_bwd_workspace_size(ctypes.byref(a))
    # packed Q^T and dO^T (300 rows padded to 320), packed K^T (200 -> 256), -D and nl per row
    assert need >= 2 * 4 * 128 * 320 * 2 + 2 * 128 * 256 * 2 + 2 * 4 * 300 * 4
    assert lib.ra_block_bwd(ctypes.byref(a), None, need, None) == 5
    assert lib.ra_block_bwd(ctypes.byref(a), ctypes.c_void_p(4096), need - 1, None) == 5
    assert lib.ra_block_bwd(ctypes.byref(a), ctypes.c_void_p(4096 + 16), need, None) == 5
    # no query rows: nothing to do, no workspace or tensors needed
    e = _block_bwd(n_q=0, q=0, o=0, dout=0, lse=0, dq=0)
    assert lib.ra_block_bwd(ctypes.byref(e), None, 0, None) == 0


def _ring_bwd(**kw):
    a = rb.RingBwdArgs()
    for f in ("q_sh", "k_sh", "v_sh", "o_sh", "dout_sh", "lse", "dq_sh", "dk_sh", "dv_sh"):
        setattr(a, f, 4096)
    a.dtype, a.R, a.rank0, a.n_ranks = rb.DT_BF16, 8, 0, 8
    a.B, a.Hq, a.Hkv, a.n, a.d = 1, 4, 2, 256, 128
    a.scale, a.causal, a.layout = 0.088, 1, rb.LAYOUT_STRIPED
    a.handoff = rb.HANDOFF_COPY
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("dtype", rb.DT_FP32, 6), ("dtype", 9, 3), ("layout", 5, 1), ("handoff", 3, 1),
    ("R", 0, 2), ("n_ranks", 9, 2),
    ("rank0", 1, 2), ("d", 32, 2), ("Hkv", 3, 2), ("n", (1 << 23) + 2, 6),
    ("scale", float("inf"), 1), ("dout_sh", 0, 1), ("lse", 0, 1), ("dv_sh", 4104, 4),
])
def test_ring_bwd_rejects(lib, field, value, status):
    a = _ring_bwd(**{field: value})
    st = lib.ra_ring_bwd(ctypes.byref(a), ctypes.c_void_p(4096), 1 << 40, None, None)
    assert st == status, (st, rb.last_error())
    assert lib.ra_ring_bwd_workspace_size(ctypes.byref(a)) == 0


def test_ring_bwd_zigzag_needs_even_blocks_and_workspace(lib):
    odd = _ring_bwd(layout=rb.LAYOUT_ZIGZAG, n=255)
    assert lib.ra_ring_bwd(ctypes.byref(odd), ctypes.c_void_p(4096), 1 << 40, None, None) == 2
    a = _ring_bwd()
    need = lib.ra_ring_bwd_workspace_size(ctypes.byref(a))
    rows = 8 * 1 * 4 * 256
    # fp32 dq of the computed rows and dk, dv of every block, plus the per-row -D and nl
    assert need >= rows * 128 * 4 + 2 * 8 * 1 * 2 * 256 * 128 * 4 + 2 * rows * 4
    assert lib.ra_ring_bwd(ctypes.byref(a), None, need, None, None) == 5
    assert lib.ra_ring_bwd(ctypes.byref(a), ctypes.c_void_p(4096), need - 1, None, None) == 5
    assert lib.ra_ring_bwd(ctypes.byref(a), ctypes.c_void_p(4096 + 16), need, None, None) == 5
    # COPY adds two receive buffers per computed rank: K, V, transposed K (16-bit) and the
    # fp32 dK, dV accumulators that travel with the block
    swap = _ring_bwd(handoff=rb.HANDOFF_SWAP)
    blk = 1 * 2 * 256 * 128
    assert need - lib.ra_ring_bwd_workspace_size(ctypes.byref(swap)) >= 2 * 8 * blk * (3 * 2 + 2 * 4)
    one = _ring_bwd(R=1, n_ranks=1)
    one_swap = _ring_bwd(R=1, n_ranks=1, handoff=rb.HANDOFF_SWAP)
    assert lib.ra_ring_bwd_workspace_size(ctypes.byref(one)) == \
        lib.ra_ring_bwd_workspace_size(ctypes.byref(one_swap))  # nothing travels on one rank


def test_decode_noalloc_rejects_before_any_gpu_call(lib):
    """Validation of the allocation-free decode runs on the host: bad arguments
    and partials beyond its 32 MiB device array are refused without a GPU."""
    a = rb.DecodeArgs()
    a.q = a.k = a.v = a.o = a.lse = 4096
    a.dtype, a.R, a.B, a.Hq, a.Hkv, a.nq, a.n, a.d = rb.DT_BF16, 2, 64, 64, 64, 16, 128, 128
    a.scale, a.causal, a.q_gid0 = 0.088, 1, 0
    assert lib.ra_decode_fwd_noalloc(None, None) == 1
    assert lib.ra_decode_fwd_workspace_size(ctypes.byref(a)) > 32 << 20
    assert lib.ra_decode_fwd_noalloc(ctypes.byref(a), None) == 6
    a.d = 96
    assert lib.ra_decode_fwd_noalloc(ctypes.byref(a), None) == 2
