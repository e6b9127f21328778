#!/usr/bin/env python3
"""Benchmark of the ring-attention path on one MI355X.

A step is one full pass of the path over one batch of synthetic input:
index maps -> shard gather of Q, K, V -> R hops of block attention folded by
online softmax, with the K/V hand-off copied on a side stream -> scatter of O
and LSE back to the original token order.  The default workload is one rank's
share of a 1M-token causal context: rank 3 of an 8-rank striped ring,
131072 queries x 8 K/V blocks of 131072 keys, Hq = Hkv = 8, d = 128, bf16.

Prints ONE JSON line (rank 0).  value = causal attention TFLOP/s with the
metric's FLOP count (4*B*H*Sq*Sk*d, halved for causal) over the measured step
time; roofline = the block-attention kernel's algorithmic FLOPs per launch over
its average launch time (HIP events recorded around every launch by the
library's timing hook, on the compute stream); cpu_baseline = the fp64 oracle
on a bounded sample of the same workload's query rows, on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA


def traffic_from_profile(kernel_sources, summary):
    """HBM bytes per block-kernel launch from the committed counter summary, or
    None when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, summary)) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for rel in kernel_sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != prof.get("kernel_sources_sha256"):
        return None
    return float(prof["hbm_bytes_per_launch"])


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_name(w, fused=True, forwards=False):
    """The block kernel a ring of this workload runs (fused: running state, else exact-max
    partials for ra_merge)."""
    if w.dtype == "fp32":
        return "attn_block32_kernel<%d>" % w.d
    name = ("attn_lean64_kernel<%s%s>" % (w.dtype, "" if fused else ", exact") if w.d == 64 else
            "attn_packed_kernel<%d,%s%s>" % (w.d, w.dtype, "" if fused else ", exact"))
    return name + (" (forwarding)" if forwards else "")


def forwards_in_kernel(rb, w, handoff):
    """Whether the ring's block kernel writes the blocks on itself (the FORWARD hand-off on
    hops too short for the thin side copy; the library's rule, ra_handoff_thin)."""
    if handoff != "forward" or w.R == 1 or w.dtype == "fp32":
        return False
    elt = 2
    kb = w.ranks * w.B * w.Hkv * w.n * w.d * elt
    vb = w.ranks * w.B * w.Hkv * w.d * ((w.n + 63) // 64 * 64) * elt
    pairs = w.ranks * w.B * w.Hq * float(w.n) * w.n * (0.5 if w.causal else 1.0)
    return not rb.thin_handoff(2.0 * (kb + vb), pairs, w.d)


def hop_forward_bytes(w):
    """Bytes a forwarding launch writes on at each hop: the K block and the packed V block of
    every computed rank whose successor is computed (on a full ring every rank; the last hop
    forwards nothing)."""
    elt = 2
    blk = w.B * w.Hkv * (w.n * w.d + w.d * ((w.n + 63) // 64 * 64)) * elt
    senders = w.ranks if w.ranks == w.R else w.ranks - 1
    return [blk * senders if h + 1 < w.R else 0 for h in range(w.R)]


def rank_hop_pairs(w, layout_code, r, h):
    """Allowed (query, key) pairs per head of computed rank r at hop h."""
    n, R = w.n, w.R
    s = (r - h) % R
    if not w.causal:
        return n * n
    if layout_code == 0:  # contiguous: past block full, own block triangle, future none
        return n * n if s < r else (n * (n + 1) // 2 if s == r else 0)
    if layout_code == 1:  # striped: key j allowed iff j*R+s <= i*R+r
        return n * (n + 1) // 2 if s <= r else n * (n - 1) // 2
    c = n // 2  # zig-zag: chunks {r, 2R-1-r} x {s, 2R-1-s}, c tokens each
    tot = 0
    for X in (r, 2 * R - 1 - r):
        for Y in (s, 2 * R - 1 - s):
            tot += c * c if Y < X else (c * (c + 1) // 2 if Y == X else 0)
    return tot


def hop_pairs(w, layout_code):
    """Allowed (query, key) pairs per head at each hop, summed over computed ranks."""
    return [sum(rank_hop_pairs(w, layout_code, r, h) for r in range(w.rank0, w.rank0 + w.ranks))
            for h in range(w.R)]


def hop_bytes(w, layout_code, fused):
    """Algorithmic HBM bytes of the block kernel at each hop, summed over computed ranks:
    for every rank whose block has allowed pairs, its Q shard and the K/V block read once,
    the fp32 O and the row statistics m, l written, and read back when the kernel folds
    into the running state (fused fold, every hop after the first).  A rank whose block
    has no allowed pair moves nothing."""
    elt = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    qkv = (w.Hq + 2 * w.Hkv) * w.B * w.n * w.d * elt
    state = w.B * w.Hq * w.n * (w.d + 2) * 4
    out = []
    for h in range(w.R):
        tot = 0
        for r in range(w.rank0, w.rank0 + w.ranks):
            if rank_hop_pairs(w, layout_code, r, h) > 0:
                tot += qkv + state * (2 if (fused and h > 0) else 1)
        out.append(tot)
    return out


def cpu_baseline(w, data, layout_code, seconds_target, seed=4242):
    """Time the fp64 oracle on a bounded, seeded sample of the workload's query rows."""
    import oracle
    oracle.build(force=False)
    orc = oracle.default()
    fwd, _ = orc.layout_maps(layout_code, w.S, w.R)
    n = w.n
    owned = fwd[w.rank0 * n:(w.rank0 + w.ranks) * n].astype(np.int64)
    rng = np.random.default_rng(seed)
    q32, k32, v32 = data["q32"], data["k32"], data["v32"]
    # calibrate with a few rows, then size the sample for ~seconds_target
    def run(nrows):
        # distinct tokens while the workload has enough of them (small ones repeat)
        t = rng.choice(owned, size=nrows, replace=nrows > owned.size)
        b = rng.integers(0, w.B, nrows)
        hh = rng.integers(0, w.Hq, nrows)
        qrows = q32[b, hh, t]
        keys = (t + 1) if w.causal else np.full(nrows, w.S)
        t0 = time.perf_counter()
        orc.attention_rows(qrows, b, hh, t, k32, v32, w.Hq, w.scale, w.causal)
        dt = time.perf_counter() - t0
        return dt, float(keys.sum())
    cores = orc.num_threads()
    # single-thread rate on a small sample (per-core figure), then all cores
    orc.set_threads(1)
    dt1, k1 = run(4)
    orc.set_threads(cores)
    dt0, k0 = run(max(2 * cores, 8))
    per_key = dt0 / max(k0, 1.0)
    avg_keys = (w.S / 2) if w.causal else w.S
    cap = 8192
    rows = int(max(cores, min(cap, seconds_target / (per_key * avg_keys))))
    dt, keys = run(rows)
    if dt < 0.6 * seconds_target and rows < cap:  # the small calibration ran slow: resize once
        rows = int(max(cores, min(cap, rows * seconds_target / max(dt, 1e-3))))
        dt, keys = run(rows)
    flops = 4.0 * w.d * keys
    total_pairs = w.metric_flops() / (4.0 * w.d)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
        "kind": "oracle",
        "sample": "%d seeded query rows of the same workload (all heads, tokens of the computed "
                  "rank), each against its full allowed key set: %.3g pairs in %.2f s; whole "
                  "workload extrapolates to %.0f s" % (rows, keys, dt, total_pairs / (keys / dt)),
        "pairs_per_s": keys / dt,
        "pairs_per_s_one_thread": k1 / dt1,
        "extrapolated_full_s": total_pairs / (keys / dt),
        "cpu_model": model,
    }


def merge_bench(torch, rb, rows=4 * 16 * 512 * 64, d=64, iters=20):
    """ra_merge on the short-block shapes (B=4, H=16, 512-token shards, R=64, d=64)."""
    dev = "cuda"
    o_a = torch.randn(rows, d, device=dev)
    o_b = torch.randn(rows, d, device=dev)
    m_a = torch.randn(rows, device=dev)
    m_b = torch.randn(rows, device=dev)
    l_a = torch.rand(rows, device=dev) + 0.5
    l_b = torch.rand(rows, device=dev) + 0.5
    for _ in range(3):
        rb.ra_merge(o_a, m_a, l_a, o_b, m_b, l_b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        rb.ra_merge(o_a, m_a, l_a, o_b, m_b, l_b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = (12 * d + 24) * rows
    return {"rows": rows, "d": d, "us_per_launch": ms * 1e3, "bytes_per_launch": nbytes,
            "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 /
            PEAK_HBM_GBS}


def step_parts_bench(torch, rb, ra, w, q, k, v, o, lse, iters=10):
    """The HBM-bound parts of a step, each timed alone with HIP events around `iters` calls
    (inputs resident): the index maps (8 B per token), the shard gather of Q, K, V and the
    scatter of O and LSE (each row read and written once; the 4-byte map entry per row is not
    counted), and ra_finalize of the running state (4d + 8 B read, elt*d + 4 B written per row;
    the step runs it inside ra_ring_fwd) on synthetic fp32 state of the same rows."""
    elt = q.element_size()
    d = w.d
    q_rows = ra.n_ranks * w.B * w.Hq * ra.n
    kv_rows = w.R * w.B * w.Hkv * ra.n

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    parts = {}

    def put(name, ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        parts[name] = {"ms": round(ms, 4), "bytes": int(nbytes), "GB/s": round(gbs, 1),
                       "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    put("layout_maps", timed(ra.maps), 8 * w.S)
    put("gather_qkv", timed(lambda: ra.gather(q, k, v)), 2 * elt * d * (q_rows + 2 * kv_rows))
    put("scatter_o_lse", timed(lambda: ra.scatter(o, lse)), 2 * (elt * d + 4) * q_rows)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 77)
    o_acc = torch.randn((q_rows, d), device="cuda", generator=g)
    m = torch.randn(q_rows, device="cuda", generator=g)
    l = torch.rand(q_rows, device="cuda", generator=g) + 0.5
    out = torch.empty((q_rows, d), dtype=q.dtype, device="cuda")
    lse_out = torch.empty(q_rows, device="cuda")
    put("finalize", timed(lambda: rb.ra_finalize(o_acc, m, l, out, lse_out)),
        (4 * d + 8 + elt * d + 4) * q_rows)
    del o_acc, m, l, out, lse_out
    return parts


def overlap_bench(torch, rb, RingAttention, w, layout, tdt, q, k, v, o, lse, ra_main,
                  pairs=5):
    """How much of the K/V hand-off the compute hides.  Steps with the hand-off
    (the run's mode: FORWARD -- blocks written on by the block kernel, side
    copies only for blocks entering from ranks that are not computed -- or
    COPY; with FORWARD also COPY) and with the blocks read in place (SWAP, no
    transfer) alternate, so clock drift falls on all alike; the hop copies
    alone are the library's hand-off copy of the hand-off bytes, once per hop,
    on one stream.  overlap = 1 - median(step_mode - step_swap) / copies alone."""
    runs = {"swap": RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal,
                                  w.scale, rank0=w.rank0, n_ranks=w.ranks,
                                  handoff=rb.HANDOFF_SWAP, merge_mode=ra_main.merge_mode)}
    main_mode = "forward" if ra_main.handoff == rb.HANDOFF_FORWARD else "copy"
    runs[main_mode] = ra_main
    if main_mode == "forward":
        runs["copy"] = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal,
                                     w.scale, rank0=w.rank0, n_ranks=w.ranks,
                                     handoff=rb.HANDOFF_COPY, merge_mode=ra_main.merge_mode)
    names = list(runs)
    for r in runs.values():
        r.run(q, k, v, o, lse)
    e = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * pairs)] for _ in names]
    torch.cuda.synchronize()
    for s in range(pairs):
        for j, nm in enumerate(names):
            e[j][2 * s].record()
            runs[nm].run(q, k, v, o, lse)
            e[j][2 * s + 1].record()
    torch.cuda.synchronize()
    t = {nm: np.array([e[j][2 * s].elapsed_time(e[j][2 * s + 1]) for s in range(pairs)])
         for j, nm in enumerate(names)}
    for nm in names:
        if nm != main_mode:
            del runs[nm]
    elt = 4 if w.dtype == "fp32" else 2
    k_bytes = w.ranks * w.B * w.Hkv * w.n * w.d * elt
    v_bytes = (w.ranks * w.B * w.Hkv * w.d * ((w.n + 63) // 64 * 64) * elt
               if w.dtype != "fp32" else k_bytes)
    per_hop = k_bytes + v_bytes
    # the form of the copy the ring picks for this workload (same rule as the library)
    pairs = w.ranks * w.B * w.Hq * float(w.n) * w.n * (0.5 if w.causal else 1.0)
    thin = rb.thin_handoff(2.0 * per_hop, pairs, w.d)
    src = torch.empty(per_hop, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    rb.ra_handoff_copy(dst, src, thin=thin)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(w.R - 1):
        rb.ra_handoff_copy(dst, src, thin=thin)
    c1.record()
    torch.cuda.synchronize()
    t_copies = c0.elapsed_time(c1)
    del src, dst
    moved = 2.0 * per_hop * (w.R - 1)  # read + write
    out = {"mode": main_mode}
    for nm in names:
        out["step_ms_" + nm] = round(float(np.median(t[nm])), 3)
    out.update({"copies_alone_ms": round(t_copies, 3), "copy_form": "thin" if thin else "wide",
                "bytes_per_hop": per_hop,
                "copy_GB/s": round(moved / (t_copies * 1e-3) / 1e9, 1)})
    for nm in names:
        if nm != "swap" and t_copies > 0:
            key = "overlap" if nm == main_mode else "overlap_" + nm
            out[key] = round(1.0 - float(np.median(t[nm] - t["swap"])) / t_copies, 3)
    return out


def backward_bench(torch, ra, w, layout_code, q, k, v, iters=3):
    """ra_ring_bwd after the forward ring (same shards): MFMA roofline with the
    algorithmic count of the backward, 10*d FLOP per allowed pair per query head
    (S = QK^T, dP = dO V^T, dV, dK, dQ; recomputing S and dP for dQ is not credited).
    Also how much of the backward hand-off (K, V, transposed K and the fp32 dK/dV
    accumulators travelling with each block) the compute hides: the pass with
    blocks read and accumulated in place (SWAP), and the hop copies alone."""
    from long_context_exact_block_amd import binding as rb
    tdt = q.dtype
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 7)
    dout = torch.randn(q.shape, device="cuda", generator=g).to(tdt)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ra.backward(dout, dq, dk, dv)  # warm-up, allocates the workspace

    def timed(handoffs):
        """One pass per entry of `handoffs`, in that order; the pass times."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(handoffs))]
        torch.cuda.synchronize()
        for i, hm in enumerate(handoffs):
            ra.bargs.handoff = hm
            ev[2 * i].record()
            rb_ring_bwd(ra)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(len(handoffs))])

    handoff0 = ra.bargs.handoff
    rb_ring_bwd(ra)
    handoff = None
    if handoff0 != rb.HANDOFF_SWAP and w.R > 1:  # FORWARD moves like COPY in the backward
        # passes with the hand-off and with the blocks in place alternate
        t = timed([handoff0, rb.HANDOFF_SWAP] * iters)
        ms, ms_swap = t[0::2], t[1::2]
        ra.bargs.handoff = handoff0
        kz = w.B * w.Hkv * w.n * w.d
        n_pad = (w.n + 63) // 64 * 64
        per_hop = w.ranks * (2 * kz * 2 + 2 * w.B * w.Hkv * w.d * n_pad + 2 * kz * 4)
        home = w.ranks * 2 * kz * 4
        pairs = w.ranks * w.B * w.Hq * float(w.n) * w.n * (0.5 if w.causal else 1.0)
        thin = rb.thin_handoff(2.0 * per_hop, pairs, w.d, 3.2)
        src = torch.empty(per_hop, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        rb.ra_handoff_copy(dst, src, thin=thin)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(w.R - 1):
            rb.ra_handoff_copy(dst, src, thin=thin)
        rb.ra_handoff_copy(dst, src, home, thin=thin)
        c1.record()
        torch.cuda.synchronize()
        t_copies = c0.elapsed_time(c1)
        del src, dst
        t_copy, t_swap = float(np.median(ms)), float(np.median(ms_swap))
        t_diff = float(np.median(ms - ms_swap))
        moved = 2.0 * (per_hop * (w.R - 1) + home)
        handoff = {"ms_copy": round(t_copy, 3), "ms_swap": round(t_swap, 3),
                   "copies_alone_ms": round(t_copies, 3), "copy_form": "thin" if thin else "wide",
                   "bytes_per_hop": per_hop,
                   "copy_GB/s": round(moved / (t_copies * 1e-3) / 1e9, 1),
                   "overlap": round(1.0 - t_diff / t_copies, 3) if t_copies > 0 else None}
    else:
        ms = timed([handoff0] * iters)
    pairs = sum(hop_pairs(w, layout_code))
    flops = 10.0 * w.d * w.B * w.Hq * pairs
    med = float(np.median(ms))
    tf = flops / (med * 1e-3) / 1e12
    del dout, dq, dk, dv
    return {"ms_median": round(med, 3), "ms_min": round(float(ms.min()), 3),
            "handoff": handoff,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flops": flops,
                         "kernels": "bwd_kv_kernel<dV>, bwd_kv_kernel<dK>, bwd_dq_kernel (+ packing, D, casts)"}}


def rb_ring_bwd(ra):
    from long_context_exact_block_amd import binding as rb
    rb.ra_ring_bwd(ra.bargs, ra.bworkspace, None, ra.copy_stream)


def rank_share_bench(torch, rb, RingAttention, w, iters=3):
    """Each rank's share of a ring run alone (w: causal MHA 32k, R = 8), for the
    contiguous, striped and zig-zag layouts: the measured counterpart of the
    per-rank causal work counts.  Times ra_ring_fwd for one computed rank (R hops, SWAP
    hand-off, fused fold) after its shards are gathered; device-side random
    inputs of the workload's shape."""
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 11)
    q = torch.randn(w.B, w.Hq, w.S, w.d, device="cuda", generator=g).to(tdt)
    k = torch.randn(w.B, w.Hkv, w.S, w.d, device="cuda", generator=g).to(tdt)
    v = torch.randn(w.B, w.Hkv, w.S, w.d, device="cuda", generator=g).to(tdt)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.S, device="cuda")
    out = {}
    for layout in ("contiguous", "striped", "zigzag"):
        if layout == "zigzag" and w.S % (2 * w.R):
            continue
        ms = []
        for r in range(w.R):
            ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                               rank0=r, n_ranks=1, handoff=rb.HANDOFF_SWAP)
            ra.run(q, k, v, o, lse)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
            torch.cuda.synchronize()
            e[0].record()
            for i in range(iters):
                ra.ring()
                e[i + 1].record()
            torch.cuda.synchronize()
            ms.append(float(np.median([e[i].elapsed_time(e[i + 1]) for i in range(iters)])))
            del ra
        a = np.array(ms)
        out[layout] = {"rank_ms": [round(x, 3) for x in ms],
                       "max_over_mean": round(float(a.max() / a.mean()), 4)}
    del q, k, v, o, lse
    return out


def length_sweep_bench(torch, rb, RingAttention, w, lengths, iters=3):
    """The headline shape (w: one rank's share, striped, causal) at shorter total
    lengths S, to expose cliffs as the sequence grows (the stress tier of the
    ruibaoantu accelerator-adaptation article, section 4.3).  Per S: the ring call
    (R hops, COPY hand-off, fused fold) on device-side random shards, TFLOP/s with
    the metric's FLOP count for one rank's share (4 B Hq (S/R) S d, halved causal)."""
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    out = []
    for S in lengths:
        if S % w.R or (w.layouts[0] == "zigzag" and S % (2 * w.R)):
            continue
        ra = RingAttention(w.B, w.Hq, w.Hkv, S, w.d, w.R, w.layouts[0], tdt, w.causal, w.scale,
                           rank0=w.rank0, n_ranks=w.ranks)
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed + S)
        for t in (ra.q_sh, ra.k_sh, ra.v_sh):
            t.copy_(torch.randn(t.shape, device="cuda", generator=g).to(tdt))
        ra.ring()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        torch.cuda.synchronize()
        e[0].record()
        for i in range(iters):
            ra.ring()
            e[i + 1].record()
        torch.cuda.synchronize()
        ms = float(np.median([e[i].elapsed_time(e[i + 1]) for i in range(iters)]))
        flops = 4.0 * w.B * w.Hq * (S // w.R) * w.ranks * S * w.d / (2 if w.causal else 1)
        tf = flops / (ms * 1e-3) / 1e12
        out.append({"S": S, "ms": round(ms, 3), "TFLOP/s": round(tf, 1),
                    "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del ra
    return out


def decode_bench(torch, rb, w, iters=20):
    """ra_decode_fwd on the long-context decode step (w: DecodeWorkload): nq new
    tokens against the whole KV cache, split contiguously over R ranks.  HBM
    roofline: algorithmic bytes = the cache (K and V, each key once) + Q, O, LSE."""
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    n = w.n
    q = torch.randn(w.B, w.Hq, w.nq, w.d, device="cuda", generator=g).to(tdt)
    k = torch.randn(w.R, w.B, w.Hkv, n, w.d, device="cuda", generator=g).to(tdt)
    v = torch.randn(w.R * w.B, w.Hkv, n, w.d, device="cuda", generator=g).to(tdt)
    vp = torch.empty(rb.ra_packed_v_bytes(rb.dtype_code(v), w.R * w.B, w.Hkv, n, w.d) // 2,
                     dtype=tdt, device="cuda")
    rb.ra_pack_v(v, vp)
    del v
    o = torch.empty(w.B, w.Hq, w.nq, w.d, dtype=tdt, device="cuda")
    lse = torch.empty(w.B, w.Hq, w.nq, dtype=torch.float32, device="cuda")
    a = rb.decode_args(q, k, vp, o, lse, 1.0 / math.sqrt(w.d), w.causal, w.S - w.nq)
    ws = torch.empty(rb.ra_decode_fwd_workspace_size(a), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        rb.ra_decode_fwd(a, ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(iters):
        rb.ra_decode_fwd(a, ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
    med = float(np.median(ms))
    nbytes = w.io_bytes()
    gbs = nbytes / (med * 1e-3) / 1e9
    del k, vp, ws
    return {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "cache_tokens": w.S,
            "R": w.R, "new_tokens": w.nq, "dtype": w.dtype,
            "ms_median": round(med, 4), "ms_min": round(float(ms.min()), 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_call": nbytes,
                         "kernels": "decode_kernel<128,bf16> + decode_reduce_kernel"}}


def block_only(torch, rb, w, layout, steps, warmup):
    """One hop of the workload through ra_block_fwd: the first computed rank's query shard
    against the block of the same source rank (hop 0), packed V, fresh state."""
    n, d = w.n, w.d
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    q = torch.randn(w.B, w.Hq, n, d, device="cuda", generator=g).to(tdt)
    k = torch.randn(w.B, w.Hkv, n, d, device="cuda", generator=g).to(tdt)
    v = torch.randn(w.B, w.Hkv, n, d, device="cuda", generator=g).to(tdt)
    packed = w.dtype != "fp32"
    if packed:
        vp = torch.empty(rb.ra_packed_v_bytes(rb.dtype_code(v), w.B, w.Hkv, n, d) // 2,
                         dtype=tdt, device="cuda")
        rb.ra_pack_v(v, vp)
        v = vp
    o = torch.empty(w.B, w.Hq, n, d, device="cuda")
    m = torch.empty(w.B, w.Hq, n, device="cuda")
    l = torch.empty(w.B, w.Hq, n, device="cuda")
    r = w.rank0
    contig = layout == "contiguous"
    g0, step = (r * n, 1) if contig else (r, w.R)

    def go():
        rb.ra_block_fwd(q, k, v, o, m, l, w.scale, w.causal, g0, step, g0, step, v_packed=packed)

    for _ in range(warmup):
        go()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        go()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = (n * (n + 1) // 2) if w.causal else n * n
    flops = 4.0 * d * w.B * w.Hq * pairs
    print(json.dumps({"mode": "block_only", "workload": w.name, "layout": layout, "ms": ms,
                      "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                      "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None, help="workload name (default: 1M-token share)")
    ap.add_argument("--layout", default=None)
    ap.add_argument("--handoff", default="forward", choices=["forward", "copy", "swap"])
    ap.add_argument("--merge", default="fused", choices=["fused", "separate"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge-bench", action="store_true")
    ap.add_argument("--no-bwd-bench", action="store_true",
                    help="skip the backward-ring measurement (ra_ring_bwd)")
    ap.add_argument("--no-decode-bench", action="store_true",
                    help="skip the long-context decode measurement (ra_decode_fwd)")
    ap.add_argument("--no-overlap-bench", action="store_true",
                    help="skip the hand-off overlap measurement (SWAP steps + copies alone)")
    ap.add_argument("--no-parts-bench", action="store_true",
                    help="skip timing the maps, gather, scatter and finalize alone")
    ap.add_argument("--no-length-sweep", action="store_true",
                    help="skip the headline shape at S = 8k .. 1M")
    ap.add_argument("--no-rank-bench", action="store_true",
                    help="skip timing each rank's share of the causal 32k MHA ring alone")
    ap.add_argument("--block-only", action="store_true",
                    help="time only the block kernel on one hop of the workload (query shard x "
                         "one K/V block, packed V), on seeded device-side random inputs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build emulates the ring of ranks on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_exact_block_amd import binding as rb
    from long_context_exact_block_amd import configs, inputs
    from long_context_exact_block_amd.pipeline import RingAttention

    w = configs.BY_NAME[args.workload] if args.workload else configs.SHARE_1M
    layout = args.layout or w.layouts[0]
    lcode = rb.LAYOUTS[layout]
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rb.lib()  # fail loudly if the HIP library is missing

    if args.block_only:
        block_only(torch, rb, w, layout, args.steps, args.warmup)
        return

    log("workload %s layout %s: generating inputs" % (w.name, layout))
    t0 = time.perf_counter()
    data = inputs.qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.seed, w.dtype, w.q_scale)
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]

    def dev(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).cuda()

    q, k, v = dev(data["q"]), dev(data["k"]), dev(data["v"])
    o = torch.zeros((w.B, w.Hq, w.S, w.d), dtype=tdt, device="cuda")
    lse = torch.zeros((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    ra = RingAttention(w.B, w.Hq, w.Hkv, w.S, w.d, w.R, layout, tdt, w.causal, w.scale,
                       rank0=w.rank0, n_ranks=w.ranks,
                       handoff={"forward": rb.HANDOFF_FORWARD, "copy": rb.HANDOFF_COPY,
                                "swap": rb.HANDOFF_SWAP}[args.handoff],
                       merge_mode=rb.MERGE_FUSED if args.merge == "fused" else rb.MERGE_SEPARATE)
    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        ra.run(q, k, v, o, lse)
    torch.cuda.synchronize()

    # per-launch timing of the block kernel through the library's hook
    R, K = w.R, args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * R * K)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    handles = [(ctypes.c_void_p * (2 * R))(*[evs[s * 2 * R + i].cuda_event for i in range(2 * R)])
               for s in range(K)]
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    log("timing %d steps" % K)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    step_ev[0].record()
    for s in range(K):
        ra.args.hop_events = ctypes.cast(handles[s], ctypes.POINTER(ctypes.c_void_p))
        ra.run(q, k, v, o, lse)
        step_ev[s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ra.args.hop_events = None
    ms_per_step = wall / K * 1e3
    step_ms = np.array([step_ev[s].elapsed_time(step_ev[s + 1]) for s in range(K)])
    hop_ms = np.array([[evs[s * 2 * R + 2 * h].elapsed_time(evs[s * 2 * R + 2 * h + 1])
                        for h in range(R)] for s in range(K)])
    pairs = hop_pairs(w, lcode)
    flops_per_launch = [4.0 * w.d * w.B * w.Hq * p for p in pairs]
    achieved = sum(flops_per_launch) * K / (hop_ms.sum() * 1e-3) / 1e12
    bytes_per_launch = hop_bytes(w, lcode, args.merge == "fused")
    # with the FORWARD hand-off on short hops the launch also writes the block on
    forwards = forwards_in_kernel(rb, w, args.handoff)
    fwd_bytes = hop_forward_bytes(w) if forwards else [0] * R
    bytes_per_launch = [a + b for a, b in zip(bytes_per_launch, fwd_bytes)]
    achieved_gbs = sum(bytes_per_launch) * K / (hop_ms.sum() * 1e-3) / 1e9
    peak_dt = PEAK_BF16_TFLOPS if w.dtype != "fp32" else PEAK_FP32_TFLOPS
    # the kernel's roof: MFMA time or HBM time of its algorithmic work, whichever is longer
    hbm_bound = sum(bytes_per_launch) / (PEAK_HBM_GBS * 1e9) > sum(flops_per_launch) / (peak_dt * 1e12)
    value = w.metric_flops() / (ms_per_step * 1e-3) / 1e12
    exact_flops = 4.0 * w.d * w.B * w.Hq * sum(pairs)
    log("step %.2f ms, %.1f TFLOP/s; block kernel %.1f TFLOP/s" % (ms_per_step, value, achieved))

    handoff = None
    if args.handoff != "swap" and w.R > 1 and not args.no_overlap_bench:
        handoff = overlap_bench(torch, rb, RingAttention, w, layout, tdt, q, k, v, o, lse, ra)
    merge = None if args.no_merge_bench else merge_bench(torch, rb)
    parts = None
    if not args.no_parts_bench:
        log("maps, gather, scatter, finalize alone")
        parts = step_parts_bench(torch, rb, ra, w, q, k, v, o, lse)
    backward = None
    if not args.no_bwd_bench and w.dtype != "fp32":
        log("backward")
        backward = backward_bench(torch, ra, w, lcode, q, k, v)
    decode = None if args.no_decode_bench else decode_bench(torch, rb, configs.DECODE_1M)
    sweep = None
    if not args.no_length_sweep and w.name == configs.SHARE_1M.name:
        log("length sweep")
        sweep = length_sweep_bench(torch, rb, RingAttention, w,
                                   [1 << e for e in range(13, 21)])
    rank_share = None
    if not args.no_rank_bench:
        log("rank shares of %s alone" % configs.MHA_32K.name)
        rank_share = rank_share_bench(torch, rb, RingAttention, configs.MHA_32K)
    imbalance = {}
    for name, code in (("contiguous", 0), ("striped", 1), ("zigzag", 2)):
        if code == 2 and w.S % (2 * w.R):
            continue
        W = rb.ra_causal_work(code, w.S, w.R)
        imbalance[name] = float(W.max() / W.mean())

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(w, data, lcode, args.cpu_seconds)

    traffic = None
    if w.name == "rank3_of_8_share_1M_striped_bf16" and args.merge == "fused":
        traffic = traffic_from_profile(
            ["long_context_exact_block_amd/csrc/block_fwd_packed.hip",
             "long_context_exact_block_amd/csrc/attn_common.h"],
            "profiles/attn_packed_1M_share_traffic.json")

    line = {
        "metric": "causal ring-attention fwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.name if layout in w.name else w.name.replace(w.layouts[0], layout),
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "S": w.S,
                   "R": w.R, "layout": layout, "causal": w.causal, "query_ranks":
                   list(range(w.rank0, w.rank0 + w.ranks)), "handoff": args.handoff,
                   "merge": args.merge},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "exact_pair_tflops": round(exact_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline": dict(
            ({"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
              "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4),
              "mfma_view": {"achieved": round(achieved, 3), "peak": peak_dt, "unit": "TFLOP/s",
                            "frac": round(achieved / peak_dt, 4)}}
             if hbm_bound else
             {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak_dt,
              "unit": "TFLOP/s", "frac": round(achieved / peak_dt, 4),
              "hbm_view": {"achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4)}}),
            traffic=traffic, kernel=kernel_name(w, args.merge == "fused", forwards),
            launches=R * K, avg_launch_ms=round(float(hop_ms.mean()), 4),
            algorithmic_flops_per_launch=sum(flops_per_launch) / R,
            algorithmic_bytes_per_launch=sum(bytes_per_launch) / R,
            handoff_bytes_per_launch=sum(fwd_bytes) / R),
        "step_ms_median": round(float(np.median(step_ms)), 3),
        "step_ms_min": round(float(step_ms.min()), 3),
        "hop_ms": [round(float(x), 3) for x in hop_ms.mean(axis=0)],
        "handoff": handoff,
        "merge": (None if merge is None else dict(merge, traffic=traffic_from_profile(
            ["long_context_exact_block_amd/csrc/elementwise.hip"], "profiles/merge_traffic.json"))),
        "step_parts": parts,
        "backward": backward,
        "decode": decode,
        "length_sweep": sweep,
        "causal_imbalance_max_over_mean": imbalance,
        "rank_share_alone": (None if rank_share is None else
                             {"workload": configs.MHA_32K.name, **rank_share}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
