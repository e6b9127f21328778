"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each ``check_*`` takes an oracle binding and raises AssertionError when the
oracle disagrees with the pinned fact.  ``test_oracle_pins.py`` runs them on
the committed oracle; ``test_oracle_mutants.py`` plants plausible mistakes in
copies of the oracle source and shows that each one trips at least one pin.

Page citations (page title and section):
* [ZZ] highthink.cn repost of the context-parallelism / Ring Attention article,
  section "Zig Zag Ring Attention 通信和计算重叠";
* [DE] aiunderstanding.org "Sequenzparallelität und Ringaufmerksamkeit",
  sections "Tiefer Einblick" and FAQ;
* [TH] Thai version of that guide, technical-insight section.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CONTIGUOUS, STRIPED, ZIGZAG = 0, 1, 2


# --------------------------------------------------------------------------- helpers
def _rng(seed):
    return np.random.default_rng(seed)


def brute_head(q, k, v, scale, causal):
    """Pure-Python exact-as-possible attention for one head (math.fsum, math.exp).

    q, k, v are lists of lists of floats [S][d].  Returns (O rows, LSE list).
    """
    S = len(q)
    d = len(q[0])
    outs, lses = [], []
    for i in range(S):
        allowed = list(range(i + 1)) if causal else list(range(S))
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in allowed]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        lsum = math.fsum(p)
        outs.append([math.fsum(p[t] * v[j][c] for t, j in enumerate(allowed)) / lsum
                     for c in range(d)])
        lses.append(m + math.log(lsum))
    return outs, lses


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ok = np.isclose(a, b, rtol=rtol, atol=atol) | ((a == b) & np.isinf(a))
    if not ok.all():
        diff = np.abs(np.nan_to_num(a - b, nan=np.inf))
        raise AssertionError("%s: max |diff| %.3e" % (what, diff.max()))


def read_interleave_golden():
    """Parse tests/golden/interleave_r4.txt -> (R, {rank: [tokens]})."""
    R = None
    ranks = {}
    with open(os.path.join(GOLDEN, "interleave_r4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("R "):
                R = int(line.split()[1])
            elif line.startswith("rank"):
                head, toks = line.split(":")
                ranks[int(head.split()[1])] = [int(t) for t in toks.split()]
    return R, ranks


def closed_form_counts(layout, S, R):
    """Per-rank causal pairs: contiguous r*n^2 + n(n+1)/2; striped R n^2/2 + n(2r+2-R)/2;
    zig-zag (chunks r and 2R-1-r of c = S/2R tokens) c^2 (2R-1) + c(c+1) for every rank."""
    n = S // R
    if layout == CONTIGUOUS:
        return np.array([r * n * n + n * (n + 1) // 2 for r in range(R)], np.int64)
    if layout == ZIGZAG:
        c = n // 2
        return np.full(R, c * c * (2 * R - 1) + c * (c + 1), np.int64)
    return np.array([(R * n * n + n * (2 * r + 2 - R)) // 2 for r in range(R)], np.int64)


def layouts_for(S, R):
    """Layouts that split S tokens over R ranks (zig-zag needs 2R equal chunks)."""
    return (CONTIGUOUS, STRIPED, ZIGZAG) if S % (2 * R) == 0 else (CONTIGUOUS, STRIPED)


# --------------------------------------------------------------------------- PIN-1
def check_layout_golden(orc):
    """[ZZ] worked example: with four ranks, rank 0 holds 0,4,8...; rank 1 holds 1,5,9..."""
    R, ranks = read_interleave_golden()
    for S in (12, 16, 64):
        fwd, _ = orc.layout_maps(STRIPED, S, R)
        n = S // R
        for r, toks in ranks.items():
            got = list(fwd[r * n: r * n + len(toks)])
            assert got == toks, (S, r, got, toks)


def check_layout_bijection(orc):
    """Both maps are bijections with inv(fwd(p)) = p; contiguous is the identity;
    every striped slot holds a token congruent to its rank mod R."""
    for S, R in ((12, 4), (1024, 4), (48, 3), (64, 64), (7, 1), (32768, 8)):
        n = S // R
        for layout in (CONTIGUOUS, STRIPED):
            fwd, inv = orc.layout_maps(layout, S, R)
            assert sorted(fwd.tolist()) == list(range(S))
            assert (inv[fwd] == np.arange(S)).all()
            assert (fwd[inv] == np.arange(S)).all()
            if layout == CONTIGUOUS:
                assert (fwd == np.arange(S)).all()
            else:
                p = np.arange(S)
                assert (fwd % R == p // n).all()          # owner rank
                assert (fwd // R == p % n).all()          # local position
                # within a rank tokens increase, so masks stay monotone
                assert (np.diff(fwd.reshape(R, n), axis=1) > 0).all()


def check_zigzag_layout(orc):
    """Zig-zag reading (2R chunks, rank r holds chunk r then chunk 2R-1-r): the
    four-rank, 16-token assignment written out by hand; bijection; each rank's
    tokens increase (causal masks stay prefixes); one early and one late chunk."""
    fwd, inv = orc.layout_maps(ZIGZAG, 16, 4)
    assert fwd.reshape(4, 4).tolist() == [[0, 1, 14, 15], [2, 3, 12, 13], [4, 5, 10, 11],
                                          [6, 7, 8, 9]]
    for S, R in ((16, 4), (48, 3), (64, 8), (2, 1), (4096, 8), (128, 64)):
        fwd, inv = orc.layout_maps(ZIGZAG, S, R)
        n, c = S // R, S // (2 * R)
        assert sorted(fwd.tolist()) == list(range(S))
        assert (inv[fwd] == np.arange(S)).all()
        f = fwd.reshape(R, n).astype(np.int64)
        assert (np.diff(f, axis=1) > 0).all()
        for r in range(R):
            assert (f[r, :c] == r * c + np.arange(c)).all()
            assert (f[r, c:] == (2 * R - 1 - r) * c + np.arange(c)).all()
    for S, R in ((12, 4), (10, 4)):  # not 2R equal chunks
        try:
            orc.layout_maps(ZIGZAG, S, R)
        except ValueError:
            continue
        raise AssertionError("zig-zag accepted S=%d R=%d" % (S, R))


# --------------------------------------------------------------------------- PIN-2
def check_brute_force(orc):
    """Oracle = pure-Python fsum brute force on tiny inputs (MHA and GQA, both masks)."""
    rng = _rng(11)
    B, Hq, Hkv, S, d = 2, 4, 2, 9, 5
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    for causal in (True, False):
        o, lse = orc.attention_full(q, k, v, scale, causal)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                bo, bl = brute_head(q[b, h].astype(np.float64).tolist(),
                                    k[b, g].astype(np.float64).tolist(),
                                    v[b, g].astype(np.float64).tolist(), scale, causal)
                _close(o[b, h], bo, 1e-13, 1e-14, "brute O")
                _close(lse[b, h], bl, 1e-13, 1e-14, "brute LSE")


def check_block_partial_brute(orc):
    """One block with affine global ids against brute force over the allowed subset;
    rows that see no key give (0, -inf, 0)."""
    rng = _rng(12)
    B, Hq, Hkv, nq, nk, d = 1, 2, 1, 6, 7, 4
    q = rng.standard_normal((B, Hq, nq, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, nk, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, nk, d)).astype(np.float32)
    scale = 0.7
    # striped-like ids: query rank 1, key source 2, R = 4 -> key j allowed iff 4j+2 <= 4i+1
    qg0, qs, kg0, ks = 1, 4, 2, 4
    o, m, l = orc.block_partial(q, k, v, scale, True, qg0, qs, kg0, ks)
    for h in range(Hq):
        for i in range(nq):
            allowed = [j for j in range(nk) if kg0 + j * ks <= qg0 + i * qs]
            if not allowed:
                assert (o[0, h, i] == 0).all() and m[0, h, i] == -math.inf and l[0, h, i] == 0
                continue
            s = [scale * math.fsum(float(q[0, h, i, c]) * float(k[0, 0, j, c]) for c in range(d))
                 for j in allowed]
            mm = max(s)
            p = [math.exp(x - mm) for x in s]
            ll = math.fsum(p)
            oo = [math.fsum(p[t] * float(v[0, 0, j, c]) for t, j in enumerate(allowed)) / ll
                  for c in range(d)]
            _close(o[0, h, i], oo, 1e-13, 1e-14, "block O")
            _close(m[0, h, i], mm, 1e-14, 1e-15, "block m")
            _close(l[0, h, i], ll, 1e-13, 1e-15, "block l")
    # row 0 of this block has no allowed key (4*0+2 > 4*0+1)
    assert m[0, 0, 0] == -math.inf


# --------------------------------------------------------------------------- PIN-3..6
def check_identical_keys(orc):
    """All keys equal: O_i = mean of the allowed values (prefix mean when causal),
    LSE_i = scale <q_i, k> + ln(#allowed)."""
    rng = _rng(13)
    B, H, S, d = 1, 2, 33, 8
    q = rng.standard_normal((B, H, S, d)).astype(np.float32)
    kv = rng.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(kv, (B, H, S, d)).copy()
    v = rng.standard_normal((B, H, S, d)).astype(np.float32)
    scale = 0.3
    for causal in (True, False):
        o, lse = orc.attention_full(q, k, v, scale, causal)
        v64 = v.astype(np.float64)
        cnt = np.arange(1, S + 1) if causal else np.full(S, S)
        if causal:
            mean = np.cumsum(v64, axis=2) / cnt[None, None, :, None]
        else:
            mean = np.broadcast_to(v64.mean(axis=2, keepdims=True), v64.shape)
        _close(o, mean, 1e-12, 1e-13, "identical-keys O")
        expect = scale * (q.astype(np.float64) @ kv.astype(np.float64)) + np.log(cnt)[None, None]
        _close(lse, expect, 1e-12, 1e-13, "identical-keys LSE")


def check_dominant_logit(orc):
    """One allowed logit beats all others by >= 40: O = that value row within
    #A e^-40 max|v|, LSE = that logit within the same bound."""
    rng = _rng(14)
    S, d = 40, 16
    scale = 0.25
    q = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    k = (0.01 * rng.standard_normal((1, 1, S, d))).astype(np.float32)
    v = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    t = S - 1
    jstar = 17
    qq = q[0, 0, t].astype(np.float64)
    k[0, 0, jstar] = (qq * (50.0 / (scale * qq @ qq))).astype(np.float32)
    o, lse = orc.attention_rows(q[0, 0, t:t + 1], [0], [0], [t], k, v, 1, scale, True)
    sstar = scale * float(q[0, 0, t].astype(np.float64) @ k[0, 0, jstar].astype(np.float64))
    others = scale * (k[0, 0, :t + 1].astype(np.float64) @ qq)
    others = np.delete(others, jstar)
    gap = sstar - others.max()
    assert gap >= 40, gap
    bound = (t + 1) * math.exp(-gap) * np.abs(v).max()
    assert np.abs(o[0] - v[0, 0, jstar]).max() <= bound + 1e-15
    assert abs(lse[0] - sstar) <= (t + 1) * math.exp(-gap) + 1e-13


def check_constant_values(orc):
    """All value rows equal c: O_i = c for every row (normalisation)."""
    rng = _rng(15)
    B, Hq, Hkv, S, d = 1, 4, 2, 50, 8
    q = (3 * rng.standard_normal((B, Hq, S, d))).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    c = rng.standard_normal(d).astype(np.float32)
    v = np.broadcast_to(c, (B, Hkv, S, d)).copy()
    for causal in (True, False):
        o, _ = orc.attention_full(q, k, v, 0.35, causal)
        _close(o, np.broadcast_to(c.astype(np.float64), o.shape), 1e-13, 1e-14, "const-V O")


def check_key_shift(orc):
    """k_j -> k_j + u for all j leaves O unchanged and shifts LSE_i by scale <q_i, u>.
    Small-integer inputs keep k + u exact in float32."""
    rng = _rng(16)
    B, H, S, d = 1, 2, 24, 8
    q = rng.integers(-3, 4, (B, H, S, d)).astype(np.float32)
    k = rng.integers(-3, 4, (B, H, S, d)).astype(np.float32)
    v = rng.standard_normal((B, H, S, d)).astype(np.float32)
    u = rng.integers(-2, 3, d).astype(np.float32)
    scale = 0.25
    for causal in (True, False):
        o1, l1 = orc.attention_full(q, k, v, scale, causal)
        o2, l2 = orc.attention_full(q, k + u, v, scale, causal)
        _close(o2, o1, 1e-12, 1e-13, "shift O")
        shift = scale * (q.astype(np.float64) @ u.astype(np.float64))
        _close(l2, l1 + shift, 1e-12, 1e-12, "shift LSE")


# --------------------------------------------------------------------------- PIN-7
def check_library_sdpa(orc):
    """R = 1 is plain attention: O against torch's scaled_dot_product_attention in
    float64 on the CPU (grouped heads by repeating K/V), LSE against scipy's
    logsumexp over the masked logits."""
    import torch
    from scipy.special import logsumexp
    rng = _rng(17)
    B, Hq, Hkv, S, d = 2, 4, 2, 37, 16
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    rep = Hq // Hkv
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double().repeat_interleave(rep, dim=1)
    tv = torch.from_numpy(v).double().repeat_interleave(rep, dim=1)
    for causal in (True, False):
        o, lse = orc.attention_full(q, k, v, scale, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=scale).numpy()
        _close(o, ref, 1e-11, 1e-12, "sdpa O")
        logits = scale * np.matmul(tq.numpy(), np.swapaxes(tk.numpy(), -1, -2))
        if causal:
            logits = np.where(np.tril(np.ones((S, S), bool)), logits, -np.inf)
        _close(lse, logsumexp(logits, axis=-1), 1e-12, 1e-12, "scipy LSE")


# --------------------------------------------------------------------------- PIN-8/9
def check_ring_equals_full(orc):
    """[DE] FAQ / [TH]: the blockwise online-softmax ring equals full attention,
    for every ring size and both layouts (fp64, up to rounding)."""
    rng = _rng(18)
    B, Hq, Hkv, S, d = 1, 2, 1, 48, 8
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    for causal in (True, False):
        o, lse = orc.attention_full(q, k, v, scale, causal)
        for R in (1, 2, 3, 4, 8, 16, 48):
            for layout in layouts_for(S, R):
                ro, rl = orc.ring_emulate(q, k, v, R, layout, scale, causal)
                _close(ro, o, 1e-12, 1e-13, "ring O R=%d L=%d" % (R, layout))
                _close(rl, lse, 1e-12, 1e-13, "ring LSE R=%d L=%d" % (R, layout))


def check_layout_independence(orc):
    """Striped and contiguous rings give the same result in the original order."""
    rng = _rng(19)
    B, H, S, d = 2, 2, 64, 4
    q = rng.standard_normal((B, H, S, d)).astype(np.float32)
    k = rng.standard_normal((B, H, S, d)).astype(np.float32)
    v = rng.standard_normal((B, H, S, d)).astype(np.float32)
    for R in (4, 8):
        a = orc.ring_emulate(q, k, v, R, CONTIGUOUS, 0.5, True)
        for layout in (STRIPED, ZIGZAG):
            b = orc.ring_emulate(q, k, v, R, layout, 0.5, True)
            _close(a[0], b[0], 1e-12, 1e-13, "layouts O")
            _close(a[1], b[1], 1e-12, 1e-13, "layouts LSE")


# --------------------------------------------------------------------------- PIN-10
def check_merge_algebra(orc):
    """(+) is commutative, associative to rounding, has identity (0, -inf, 0), and
    folding the partials of any partition of a row's keys gives the full row."""
    rng = _rng(20)
    rows, d = 16, 8

    def part(seed):
        r = _rng(seed)
        return (r.standard_normal((rows, d)), r.standard_normal(rows) * 3,
                np.exp(r.standard_normal(rows)))

    a, b, c = part(1), part(2), part(3)
    ab = orc.merge(*a, *b)
    ba = orc.merge(*b, *a)
    for x, y in zip(ab, ba):
        assert np.array_equal(x, y)
    ab_c = orc.merge(*ab, *c)
    a_bc = orc.merge(*a, *orc.merge(*b, *c))
    for x, y in zip(ab_c, a_bc):
        _close(x, y, 1e-13, 1e-14, "assoc")
    ident = (np.zeros((rows, d)), np.full(rows, -np.inf), np.zeros(rows))
    for x, y in zip(orc.merge(*a, *ident), a):
        _close(x, y, 1e-15, 1e-15, "identity right")
    for x, y in zip(orc.merge(*ident, *a), a):
        _close(x, y, 1e-15, 1e-15, "identity left")
    e = orc.merge(*ident, *ident)
    assert (e[0] == 0).all() and (e[1] == -np.inf).all() and (e[2] == 0).all()
    # partition folding: keys split into uneven contiguous pieces
    B, H, S, dd = 1, 1, 30, 8
    q = rng.standard_normal((B, H, S, dd)).astype(np.float32)
    k = rng.standard_normal((B, H, S, dd)).astype(np.float32)
    v = rng.standard_normal((B, H, S, dd)).astype(np.float32)
    o_full, lse_full = orc.attention_full(q, k, v, 0.4, True)
    cuts = [0, 7, 8, 19, 30]
    acc = (np.zeros((S, dd)), np.full(S, -np.inf), np.zeros(S))
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        po, pm, pl = orc.block_partial(q, k[:, :, lo:hi], v[:, :, lo:hi], 0.4, True, 0, 1, lo, 1)
        acc = orc.merge(*acc, po[0, 0], pm[0, 0], pl[0, 0])
    _close(acc[0], o_full[0, 0], 1e-12, 1e-13, "partition O")
    _close(acc[1] + np.log(acc[2]), lse_full[0, 0], 1e-12, 1e-13, "partition LSE")


# --------------------------------------------------------------------------- PIN-11
def check_pair_counts(orc):
    """Per-rank causal pair counts: brute force equals the closed forms, sums to
    S(S+1)/2; the striped layout is balanced to within one row per block ([ZZ])."""
    for S, R in ((8, 2), (16, 4), (24, 4), (32, 8), (64, 8), (60, 6), (48, 3), (128, 16)):
        for layout in layouts_for(S, R):
            W = orc.pair_counts(layout, S, R)
            assert (W == closed_form_counts(layout, S, R)).all(), (S, R, layout, W)
            assert W.sum() == S * (S + 1) // 2
        Ws = orc.pair_counts(STRIPED, S, R)
        assert Ws.max() - Ws.min() == (R - 1) * (S // R)


def check_coverage(orc):
    """[ZZ]/[DE]: after one full loop every query has met every allowed key exactly
    once.  With all-zero Q and K every logit is 0, so e^LSE counts the keys seen."""
    B, H, S, d = 1, 1, 40, 4
    z = np.zeros((B, H, S, d), np.float32)
    v = np.ones((B, H, S, d), np.float32)
    for R in (1, 2, 4, 5, 8):
        for layout in layouts_for(S, R):
            for causal in (True, False):
                _, lse = orc.ring_emulate(z, z, v, R, layout, 1.0, causal)
                seen = np.exp(lse[0, 0])
                expect = np.arange(1, S + 1) if causal else np.full(S, S)
                _close(seen, expect, 1e-12, 1e-12, "coverage")


# --------------------------------------------------------------------------- PIN-12
def check_gqa_equals_repeated_mha(orc):
    """Grouped heads equal MHA with each K/V head repeated Hq/Hkv times (bitwise)."""
    rng = _rng(21)
    B, Hq, Hkv, S, d = 1, 8, 2, 20, 8
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    o1, l1 = orc.attention_full(q, k, v, 0.3, True)
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    o2, l2 = orc.attention_full(q, kr, vr, 0.3, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --------------------------------------------------------------------------- backward
def _brute_loss(q, k, v, g, scale, causal, group):
    """sum over rows of <dO, O> with O from the pure-Python brute force (fp64)."""
    B, Hq = len(q), len(q[0])
    total = 0.0
    for b in range(B):
        for h in range(Hq):
            o, _ = brute_head(q[b][h], k[b][h // group], v[b][h // group], scale, causal)
            total += math.fsum(g[b][h][i][c] * o[i][c] for i in range(len(o))
                               for c in range(len(o[0])))
    return total


def check_bwd_finite_differences(orc):
    """The analytic gradients equal central finite differences of L = sum <dO, O>,
    with O from the pure-Python brute force in fp64, for every element of q, k, v
    (grouped heads, both masks)."""
    rng = _rng(31)
    B, Hq, Hkv, S, d = 1, 2, 1, 5, 3
    group = Hq // Hkv
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    g = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    scale = 0.7
    eps = 1e-5
    for causal in (True, False):
        dq, dk, dv = orc.attention_bwd(q, k, v, g, scale, causal)
        base = [x.astype(np.float64).tolist() for x in (q, k, v)]
        gl = g.astype(np.float64).tolist()
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            shape = grad.shape
            for idx in np.ndindex(*shape):
                vals = []
                for sgn in (1.0, -1.0):
                    t = [copy_nested(x) for x in base]
                    b_, h_, i_, c_ = idx
                    t[which][b_][h_][i_][c_] += sgn * eps
                    vals.append(_brute_loss(t[0], t[1], t[2], gl, scale, causal, group))
                fd = (vals[0] - vals[1]) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def copy_nested(x):
    return [copy_nested(y) for y in x] if isinstance(x, list) else x


def check_bwd_block_partition(orc):
    """Block contributions with the global lse and D = <dO, O> add up to the full
    gradients, for a partition of the keys and of the queries into uneven blocks."""
    rng = _rng(32)
    B, Hq, Hkv, S, d = 1, 4, 2, 23, 6
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    g = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    scale = 0.45
    for causal in (True, False):
        dq, dk, dv = orc.attention_bwd(q, k, v, g, scale, causal)
        o, lse = orc.attention_full(q, k, v, scale, causal)
        Dv = (g.astype(np.float64) * o).sum(-1)
        aq, ak, av = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
        qcuts, kcuts = [0, 9, 10, 23], [0, 4, 17, 23]
        for q0, q1 in zip(qcuts[:-1], qcuts[1:]):
            for k0, k1 in zip(kcuts[:-1], kcuts[1:]):
                bq, bk, bv = orc.block_bwd(q[:, :, q0:q1], k[:, :, k0:k1], v[:, :, k0:k1],
                                           g[:, :, q0:q1], lse[:, :, q0:q1], Dv[:, :, q0:q1],
                                           scale, causal, np.arange(q0, q1), np.arange(k0, k1))
                aq[:, :, q0:q1] += bq
                ak[:, :, k0:k1] += bk
                av[:, :, k0:k1] += bv
        _close(aq, dq, 1e-11, 1e-12, "partition dq")
        _close(ak, dk, 1e-11, 1e-12, "partition dk")
        _close(av, dv, 1e-11, 1e-12, "partition dv")


def check_bwd_constant_values(orc):
    """All value rows equal: O no longer depends on q or k, so dq = dk = 0, and
    the value gradients of a query row sum to its dO (probabilities sum to 1)."""
    rng = _rng(33)
    B, Hq, Hkv, S, d = 1, 2, 2, 9, 4
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = np.broadcast_to(rng.standard_normal(d).astype(np.float32), (B, Hkv, S, d)).copy()
    g = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    dq, dk, dv = orc.attention_bwd(q, k, v, g, 0.8, True)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    _close(dv.sum(axis=2), g.astype(np.float64).sum(axis=2), 1e-12, 1e-12, "dv sums")


def check_bwd_sampled_outputs(orc):
    """The one-output-at-a-time backward (query rows, then keys from listed rows)
    equals the whole gradient (pinned by finite differences above), both masks,
    grouped heads."""
    rng = _rng(34)
    B, Hq, Hkv, S, d = 2, 4, 2, 17, 5
    q = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    g = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    for causal in (True, False):
        dq, dk, dv = orc.attention_bwd(q, k, v, g, 0.6, causal)
        o, lse_full = orc.attention_full(q, k, v, 0.6, causal)
        bb, hh, tt = (x.ravel() for x in np.meshgrid(np.arange(B), np.arange(Hq), np.arange(S),
                                                      indexing="ij"))
        rq, rl, rD = orc.bwd_query_rows(q[bb, hh, tt], g[bb, hh, tt], bb, hh, tt, k, v, Hq, 0.6,
                                        causal)
        _close(rq.reshape(B, Hq, S, d), dq, 1e-12, 1e-13, "rows dq")
        _close(rl.reshape(B, Hq, S), lse_full, 1e-12, 1e-13, "rows lse")
        _close(rD.reshape(B, Hq, S), (g.astype(np.float64) * o).sum(-1), 1e-12, 1e-13, "rows D")
        kb, kg, kt = (x.ravel() for x in np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(S),
                                                      indexing="ij"))
        rk, rv = orc.bwd_keys(q[bb, hh, tt], g[bb, hh, tt], bb, hh, tt, rl, rD, kb, kg, kt, k, v,
                              Hq, 0.6, causal)
        _close(rk.reshape(B, Hkv, S, d), dk, 1e-12, 1e-13, "keys dk")
        _close(rv.reshape(B, Hkv, S, d), dv, 1e-12, 1e-13, "keys dv")


ALL_CHECKS = [
    check_layout_golden, check_layout_bijection, check_zigzag_layout, check_brute_force, check_block_partial_brute,
    check_identical_keys, check_dominant_logit, check_constant_values, check_key_shift,
    check_library_sdpa, check_ring_equals_full, check_layout_independence, check_merge_algebra,
    check_pair_counts, check_coverage, check_gqa_equals_repeated_mha,
    check_bwd_finite_differences, check_bwd_block_partition, check_bwd_constant_values,
    check_bwd_sampled_outputs,
]
