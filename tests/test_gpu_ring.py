"""ra_ring_fwd (the whole emulated ring) against the fp64 oracle on small and
medium shapes: every row compared; both layouts, ring sizes 1..8, a single
rank's share, grouped heads, all dtypes, causal and not.  Plus the ring's own
invariants: COPY, FORWARD and SWAP hand-offs bitwise equal, run-to-run bitwise equal,
FUSED and SEPARATE folds equal to rounding, and the original-order pipeline."""
import math

import numpy as np
import pytest

import oracle
from long_context_exact_block_amd import binding as rb
from long_context_exact_block_amd import configs, inputs
from long_context_exact_block_amd.pipeline import RingAttention
from tests import parity

pytestmark = pytest.mark.gpu

# (name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks)
CASES = [
    ("tiny_fp32_striped_R4", 1, 2, 2, 1024, 64, 4, "striped", "fp32", True, 0, 4),
    ("bf16_striped_R4_gqa", 1, 4, 2, 2048, 128, 4, "striped", "bf16", True, 0, 4),
    ("fp16_contig_R3", 1, 2, 2, 1536, 64, 3, "contiguous", "fp16", True, 0, 3),
    ("bf16_contig_R8_noncausal", 2, 2, 1, 1024, 128, 8, "contiguous", "bf16", False, 0, 8),
    ("bf16_striped_R1", 1, 2, 2, 640, 64, 1, "striped", "bf16", True, 0, 1),
    ("bf16_striped_rank3_of_8", 1, 4, 4, 4096, 128, 8, "striped", "bf16", True, 3, 1),
    ("bf16_contig_ranks1to2_of_4", 1, 2, 2, 1024, 128, 4, "contiguous", "bf16", True, 1, 2),
    ("fp16_contig_R16_short", 2, 2, 2, 2048, 64, 16, "contiguous", "fp16", False, 0, 16),
    ("bf16_striped_ragged_n", 1, 2, 2, 8 * 200, 128, 8, "striped", "bf16", True, 0, 8),
    ("fp32_contig_R2_d128", 1, 2, 1, 512, 128, 2, "contiguous", "fp32", True, 0, 2),
    ("bf16_zigzag_R4_gqa", 1, 4, 2, 2048, 128, 4, "zigzag", "bf16", True, 0, 4),
    ("fp16_zigzag_R8_d64", 2, 2, 2, 4096, 64, 8, "zigzag", "fp16", True, 0, 8),
    ("bf16_zigzag_rank5_of_8", 1, 2, 2, 8192, 128, 8, "zigzag", "bf16", True, 5, 1),
    ("bf16_zigzag_ragged_chunks", 1, 2, 2, 8 * 200, 128, 4, "zigzag", "bf16", True, 0, 4),
    ("fp32_zigzag_R3", 1, 2, 2, 768, 64, 3, "zigzag", "fp32", True, 0, 3),
    ("bf16_zigzag_noncausal", 1, 2, 2, 1024, 128, 4, "zigzag", "bf16", False, 0, 4),
    # K/V groups a multiple of 8 (one XCD per group residue): causal work taken two groups at a
    # time -- an even count of groups per XCD, an odd one (the last group alone), query heads as
    # work items of their own (3 per K/V head), and grouped heads in one workgroup
    ("bf16_striped_R2_16groups_3heads", 1, 24, 8, 1024, 64, 2, "striped", "bf16", True, 0, 2),
    ("fp16_contig_R3_24groups", 1, 8, 8, 1536, 128, 3, "contiguous", "fp16", True, 0, 3),
    ("bf16_zigzag_R2_16groups_gqa4", 1, 32, 8, 2048, 128, 2, "zigzag", "bf16", True, 0, 2),
]


def make_inputs(B, Hq, Hkv, S, d, dtype, seed, q_scale=1.0):
    x = inputs.qkv(B, Hq, Hkv, S, d, seed, dtype, q_scale)
    return x


def run_ring(case, x, handoff=rb.HANDOFF_COPY, merge_mode=rb.MERGE_FUSED, same_stream=False):
    import torch
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    ra = RingAttention(B, Hq, Hkv, S, d, R, layout, parity.torch_dtype(dtype), causal,
                       rank0=rank0, n_ranks=n_ranks, handoff=handoff, merge_mode=merge_mode,
                       copy_stream=not same_stream)
    q = parity.to_device(x["q"], dtype)
    k = parity.to_device(x["k"], dtype)
    v = parity.to_device(x["v"], dtype)
    o = torch.zeros((B, Hq, S, d), dtype=q.dtype, device="cuda")
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()
    return ra, o, lse


def owned_tokens(case):
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    fwd, _ = oracle.layout_maps(rb.LAYOUTS[layout], S, R)
    n = S // R
    return np.sort(fwd[rank0 * n:(rank0 + n_ranks) * n])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_ring_matches_oracle_all_rows(case):
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 9000 + len(name))
    _, o, lse = run_ring(case, x)
    ro, rl = oracle.attention_full(x["q32"], x["k32"], x["v32"], 1 / math.sqrt(d), causal)
    tok = owned_tokens(case)
    go = parity.to_f64(o)[:, :, tok]
    gl = parity.to_f64(lse)[:, :, tok]
    parity.check_o(go, ro[:, :, tok], name)
    parity.check_lse(gl, rl[:, :, tok], name)
    if dtype == "fp32":  # fp32 MFMA path: far inside the bound
        assert np.abs(go - ro[:, :, tok]).max() < 1e-4


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[5], CASES[6]], ids=lambda c: c[0])
def test_copy_equals_swap_and_is_deterministic(case):
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 77)
    _, o1, l1 = run_ring(case, x, rb.HANDOFF_COPY)
    _, o2, l2 = run_ring(case, x, rb.HANDOFF_SWAP)
    _, o3, l3 = run_ring(case, x, rb.HANDOFF_COPY)
    _, o4, l4 = run_ring(case, x, rb.HANDOFF_COPY, same_stream=True)
    import torch
    # rows of ranks that are not computed stay NaN in every run
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o1, o)
        assert torch.equal(torch.nan_to_num(l1, nan=7.0), torch.nan_to_num(l, nan=7.0))


# FORWARD on full rings (the block kernels write every block on: d = 128 and the
# lean d = 64 kernel, grouped heads with one workgroup per group and with one
# per head, ragged tiles, contiguous causal hops whose workgroups have no keys
# and only forward), on rank subsets (side copy for the entering block) and on
# the fp32 path (copied as in COPY)
FWD_CASES = [CASES[i] for i in (0, 1, 2, 3, 5, 6, 7, 8, 10, 11, 12)] + [
    ("bf16_striped_R4_gqa3", 1, 3, 1, 1024, 128, 4, "striped", "bf16", True, 0, 4),
    ("bf16_contig_R4_causal", 1, 2, 2, 2048, 128, 4, "contiguous", "bf16", True, 0, 4),
    ("fp16_contig_R4_d64_ranks0to2", 1, 4, 2, 2048, 64, 4, "contiguous", "fp16", True, 0, 3),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c[0])
def test_forward_equals_swap(case):
    """FORWARD hand-off: the block kernel writes each block it streams to the next
    computed rank's receive buffer.  Bitwise equal to SWAP in both folds, with one
    stream or two."""
    import torch
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 83)
    for mm in (rb.MERGE_FUSED, rb.MERGE_SEPARATE):
        _, o0, l0 = run_ring(case, x, rb.HANDOFF_SWAP, merge_mode=mm)
        for same in (False, True):
            _, o1, l1 = run_ring(case, x, rb.HANDOFF_FORWARD, merge_mode=mm, same_stream=same)
            # rows of ranks that are not computed stay NaN in every run
            assert torch.equal(o0, o1), (name, mm, same)
            assert torch.equal(torch.nan_to_num(l0, nan=7.0), torch.nan_to_num(l1, nan=7.0)), (
                name, mm, same)


@pytest.mark.parametrize("case", [FWD_CASES[i] for i in (1, 2, 6)], ids=lambda c: c[0])
def test_forward_matches_oracle(case):
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 84)
    _, o, lse = run_ring(case, x, rb.HANDOFF_FORWARD)
    ro, rl = oracle.attention_full(x["q32"], x["k32"], x["v32"], 1 / math.sqrt(d), causal)
    tok = owned_tokens(case)
    parity.check_o(parity.to_f64(o)[:, :, tok], ro[:, :, tok], name)
    parity.check_lse(parity.to_f64(lse)[:, :, tok], rl[:, :, tok], name)


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3], CASES[7]], ids=lambda c: c[0])
def test_fused_and_separate_merge_agree(case):
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 78)
    _, o1, l1 = run_ring(case, x, merge_mode=rb.MERGE_FUSED)
    _, o2, l2 = run_ring(case, x, merge_mode=rb.MERGE_SEPARATE)
    ro, rl = oracle.attention_full(x["q32"], x["k32"], x["v32"], 1 / math.sqrt(d), causal)
    tok = owned_tokens(case)
    for o, l in ((o1, l1), (o2, l2)):
        parity.check_o(parity.to_f64(o)[:, :, tok], ro[:, :, tok], name)
        parity.check_lse(parity.to_f64(l)[:, :, tok], rl[:, :, tok], name)
    # the two folds differ only in rounding order
    assert np.abs(parity.to_f64(o1) - parity.to_f64(o2))[:, :, tok].max() <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["striped", "contiguous"])
def test_running_max_rises_across_tiles_and_hops(dtype, layout):
    """Key magnitudes ramp over the token index (up by 13x) and queries are
    sharp, so the running maximum keeps rising in processing order: tile by
    tile inside a striped block (keys ordered by token, magnitudes growing),
    hop by hop on a contiguous ring (each hop brings an earlier block, ramp
    reversed).  The fused fold must raise it -- rescale and redo a tile --
    many times, including after tiles whose probabilities were all tiny."""
    B, Hq, Hkv, S, d, R = 1, 2, 2, 8 * 512, 128, 8
    case = ("rising_max_" + layout, B, Hq, Hkv, S, d, R, layout, dtype, True, 0, R)
    q32 = inputs.normal((B, Hq, S, d), 501, scale=2.0)
    k32 = inputs.normal((B, Hkv, S, d), 502)
    u = np.arange(S, dtype=np.float32) / S
    ramp = 1.0 + 12.0 * (u if layout == "striped" else 1.0 - u)
    k32 *= ramp[None, None, :, None]
    v32 = inputs.normal((B, Hkv, S, d), 503)
    x = {}
    for name, t in (("q", q32), ("k", k32), ("v", v32)):
        x[name], x[name + "32"] = inputs.to_dtype(t, dtype)
    _, o, lse = run_ring(case, x)
    ro, rl = oracle.attention_full(x["q32"], x["k32"], x["v32"], 1 / math.sqrt(d), True)
    parity.check_o(parity.to_f64(o), ro, case[0])
    parity.check_lse(parity.to_f64(lse), rl, case[0])


def test_layouts_agree_after_unpermuting():
    """Contiguous, striped and zig-zag rings give the same outputs in the original order."""
    x = make_inputs(1, 2, 2, 2048, 128, "bf16", 79)
    case_c = ("c", 1, 2, 2, 2048, 128, 8, "contiguous", "bf16", True, 0, 8)
    _, oc, lc = run_ring(case_c, x)
    for layout in ("striped", "zigzag"):
        _, o2, l2 = run_ring(("s", 1, 2, 2, 2048, 128, 8, layout, "bf16", True, 0, 8), x)
        assert np.abs(parity.to_f64(oc) - parity.to_f64(o2)).max() <= 2e-2
        assert np.abs(parity.to_f64(lc) - parity.to_f64(l2)).max() <= 1e-3


def test_repeated_calls_do_not_grow_memory():
    import torch
    case = CASES[1]
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 80)
    ra, o, lse = run_ring(case, x)
    q = parity.to_device(x["q"], dtype)
    k = parity.to_device(x["k"], dtype)
    v = parity.to_device(x["v"], dtype)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    ev0 = rb.ra_cached_events()
    for _ in range(100):
        ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 < (64 << 20)
    assert rb.ra_cached_events() == ev0  # each call hands its events back


def test_stream_delays_keep_results():
    """A bounded sleep on the copy stream before each hand-off, or on the compute
    stream before each hop, shifts the two streams against each other; with the
    events ordering them correctly the outputs stay bitwise equal."""
    import os
    import torch
    for case, hm in ((CASES[1], rb.HANDOFF_COPY), (CASES[5], rb.HANDOFF_COPY),
                     (CASES[7], rb.HANDOFF_COPY), (CASES[11], rb.HANDOFF_COPY),
                     (CASES[6], rb.HANDOFF_FORWARD), (CASES[7], rb.HANDOFF_FORWARD)):
        name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
        x = make_inputs(B, Hq, Hkv, S, d, dtype, 81)
        _, o0, l0 = run_ring(case, x, hm)
        for var in ("RA_DEBUG_DELAY_COPY", "RA_DEBUG_DELAY_COMPUTE"):
            os.environ[var] = "40"
            try:
                _, o1, l1 = run_ring(case, x, hm)
            finally:
                del os.environ[var]
            # rows of ranks that are not computed stay NaN in every run
            assert torch.equal(o0, o1), (name, var)
            assert torch.equal(torch.nan_to_num(l0, nan=7.0), torch.nan_to_num(l1, nan=7.0)), (
                name, var)


def test_rings_on_several_host_threads():
    """Ring calls from several host threads at once, each with its own streams,
    give the single-threaded results, and the event cache grows at most by one
    set per concurrent call."""
    import threading
    import torch
    case = CASES[1]
    name, B, Hq, Hkv, S, d, R, layout, dtype, causal, rank0, n_ranks = case
    x = make_inputs(B, Hq, Hkv, S, d, dtype, 82)
    _, o_ref, l_ref = run_ring(case, x)
    ev0 = rb.ra_cached_events()
    nthreads, calls = 4, 6
    results, errors = [None] * nthreads, []

    def worker(t):
        try:
            with torch.cuda.stream(torch.cuda.Stream()):
                ra = RingAttention(B, Hq, Hkv, S, d, R, layout, parity.torch_dtype(dtype), causal,
                                   rank0=rank0, n_ranks=n_ranks)
                q = parity.to_device(x["q"], dtype)
                k = parity.to_device(x["k"], dtype)
                v = parity.to_device(x["v"], dtype)
                o = torch.zeros_like(o_ref)
                lse = torch.zeros_like(l_ref)
                for _ in range(calls):
                    ra.run(q, k, v, o, lse, torch.cuda.current_stream())
                torch.cuda.current_stream().synchronize()
                results[t] = (o, lse)
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for o, lse in results:
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert rb.ra_cached_events() - ev0 <= nthreads * (2 * R + 2)
