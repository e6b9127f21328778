"""fp64 CPU oracle for exact attention and its ring emulation.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``long_context_exact_block_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C99, double precision, OpenMP over
independent rows); this module compiles it with gcc and marshals numpy arrays.
Every function states the definition it follows; citations name the page and
section:

* highthink.cn repost of the context-parallelism / Ring Attention article,
  section "Zig Zag Ring Attention 通信和计算重叠" -- the ring loop, the causal
  rule, and the interleaved token assignment.
* aiunderstanding.org guide "Sequenzparallelität und Ringaufmerksamkeit",
  sections "Tiefer Einblick" and the FAQ -- contiguous split, online softmax,
  blockwise result equal to full attention.
* the Thai version of that guide, technical-insight section -- running max,
  running normaliser, rescaling of earlier partial sums.

Parity pins for every function are in ``tests/test_oracle_pins.py``; none of
the functions here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CONTIGUOUS = 0
STRIPED = 1

_CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain IEEE double, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc"] + _CFLAGS + [_SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes binding of one build of oracle.c (the default build, or a test variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        D = ctypes.c_double
        C = ctypes.c_int
        lib.ora_num_threads.restype = C
        lib.ora_set_threads.argtypes = [C]
        lib.ora_layout_maps.argtypes = [C, I64, I32, P, P]
        lib.ora_layout_maps.restype = C
        lib.ora_attention_rows.argtypes = [P, P, P, P, I64, P, P, I64, I64, I64, I64, I64,
                                           D, C, P, P]
        lib.ora_block_partial.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, D, C,
                                          I64, I64, I64, I64, P, P, P]
        lib.ora_merge.argtypes = [P, P, P, P, P, P, I64, I64]
        lib.ora_ring_emulate.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, C, D, C, P,
                                         P]
        lib.ora_ring_emulate.restype = C
        lib.ora_pair_counts.argtypes = [C, I64, I32, P]
        lib.ora_pair_counts.restype = C
        lib.ora_bwd_query_rows.argtypes = [P, P, P, P, P, I64, P, P, I64, I64, I64, I64, D, C,
                                           P, P, P]
        lib.ora_bwd_keys.argtypes = [P, P, P, P, P, P, P, I64, P, P, P, I64, P, P, I64, I64, I64,
                                     I64, D, C, P, P]
        lib.ora_attention_bwd.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, D, C, P, P, P]
        lib.ora_attention_bwd.restype = C
        lib.ora_block_bwd.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, D, C, P, P,
                                      P, P, P]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.ora_num_threads())

    def set_threads(self, n: int) -> None:
        self.lib.ora_set_threads(int(n))

    def layout_maps(self, layout: int, S: int, R: int):
        """Slot p = r*n + j -> token fwd[p]; inv[fwd[p]] = p (int32)."""
        fwd = np.empty(S, np.int32)
        inv = np.empty(S, np.int32)
        rc = self.lib.ora_layout_maps(int(layout), int(S), int(R), _ptr(fwd), _ptr(inv))
        if rc != 0:
            raise ValueError("layout_maps: S must be divisible by R and layout known")
        return fwd, inv

    def attention_rows(self, q_rows, row_b, row_h, row_t, k, v, Hq: int, scale: float,
                       causal: bool):
        """Full-softmax attention of the listed query rows (original token order).

        q_rows [nrows][d]; row_b/row_h/row_t int64 [nrows]; k, v [B][Hkv][S][d].
        Returns (o [nrows][d] float64, lse [nrows] float64).
        """
        q_rows = _f32(q_rows)
        k = _f32(k)
        v = _f32(v)
        B, Hkv, S, d = k.shape
        nrows = q_rows.shape[0]
        rb = np.ascontiguousarray(row_b, np.int64)
        rh = np.ascontiguousarray(row_h, np.int64)
        rt = np.ascontiguousarray(row_t, np.int64)
        o = np.empty((nrows, d), np.float64)
        lse = np.empty(nrows, np.float64)
        self.lib.ora_attention_rows(_ptr(q_rows), _ptr(rb), _ptr(rh), _ptr(rt), nrows,
                                    _ptr(k), _ptr(v), B, Hq, Hkv, S, d, float(scale),
                                    int(bool(causal)), _ptr(o), _ptr(lse))
        return o, lse

    def attention_full(self, q, k, v, scale: float, causal: bool):
        """All rows: q [B][Hq][S][d] -> (o [B][Hq][S][d], lse [B][Hq][S]) in float64."""
        q = _f32(q)
        B, Hq, S, d = q.shape
        bb, hh, tt = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(S), indexing="ij")
        o, lse = self.attention_rows(q.reshape(-1, d), bb.ravel(), hh.ravel(), tt.ravel(), k,
                                     v, Hq, scale, causal)
        return o.reshape(B, Hq, S, d), lse.reshape(B, Hq, S)

    def block_partial(self, q, k, v, scale: float, causal: bool, qg0: int, qstep: int,
                      kg0: int, kstep: int):
        """Partial attention of a query shard against one key/value block.

        q [B][Hq][nq][d], k, v [B][Hkv][nk][d]; global ids gid0 + j*step.
        Returns (o [B][Hq][nq][d], m [B][Hq][nq], l [B][Hq][nq]) float64, with
        (0, -inf, 0) for rows that see no key of the block.
        """
        q = _f32(q)
        k = _f32(k)
        v = _f32(v)
        B, Hq, nq, d = q.shape
        _, Hkv, nk, _ = k.shape
        o = np.empty((B, Hq, nq, d), np.float64)
        m = np.empty((B, Hq, nq), np.float64)
        l = np.empty((B, Hq, nq), np.float64)
        self.lib.ora_block_partial(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, nq, nk, d,
                                   float(scale), int(bool(causal)), int(qg0), int(qstep),
                                   int(kg0), int(kstep), _ptr(o), _ptr(m), _ptr(l))
        return o, m, l

    def merge(self, o_a, m_a, l_a, o_b, m_b, l_b):
        """(O_a, m_a, l_a) (+) (O_b, m_b, l_b) for rows x d; returns new arrays."""
        o = np.array(o_a, np.float64, copy=True, order="C")
        m = np.array(m_a, np.float64, copy=True, order="C")
        l = np.array(l_a, np.float64, copy=True, order="C")
        ob = np.ascontiguousarray(o_b, np.float64)
        mb = np.ascontiguousarray(m_b, np.float64)
        lb = np.ascontiguousarray(l_b, np.float64)
        rows = m.size
        d = o.size // max(rows, 1)
        self.lib.ora_merge(_ptr(o), _ptr(m), _ptr(l), _ptr(ob), _ptr(mb), _ptr(lb), rows, d)
        return o, m, l

    def ring_emulate(self, q, k, v, R: int, layout: int, scale: float, causal: bool):
        """The ring of R ranks emulated on the CPU in fp64 (original token order)."""
        q = _f32(q)
        k = _f32(k)
        v = _f32(v)
        B, Hq, S, d = q.shape
        Hkv = k.shape[1]
        o = np.empty((B, Hq, S, d), np.float64)
        lse = np.empty((B, Hq, S), np.float64)
        rc = self.lib.ora_ring_emulate(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, S, d, int(R),
                                       int(layout), float(scale), int(bool(causal)), _ptr(o),
                                       _ptr(lse))
        if rc != 0:
            raise ValueError("ring_emulate: bad split or out of memory")
        return o, lse

    def pair_counts(self, layout: int, S: int, R: int):
        """Per-rank causal (query, key) pair counts by brute force (small S)."""
        W = np.empty(R, np.int64)
        rc = self.lib.ora_pair_counts(int(layout), int(S), int(R), _ptr(W))
        if rc != 0:
            raise ValueError("pair_counts: bad split")
        return W


    def attention_bwd(self, q, k, v, dout, scale: float, causal: bool):
        """Gradients of exact attention (original token order), float64:
        q, dout [B][Hq][S][d]; k, v [B][Hkv][S][d] -> (dq, dk, dv)."""
        q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
        B, Hq, S, d = q.shape
        Hkv = k.shape[1]
        dq = np.empty((B, Hq, S, d), np.float64)
        dk = np.empty((B, Hkv, S, d), np.float64)
        dv = np.empty((B, Hkv, S, d), np.float64)
        rc = self.lib.ora_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Hq, Hkv, S, d,
                                        float(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                                        _ptr(dv))
        if rc != 0:
            raise MemoryError("attention_bwd")
        return dq, dk, dv

    def bwd_query_rows(self, q_rows, dout_rows, row_b, row_h, row_t, k, v, Hq: int,
                       scale: float, causal: bool):
        """dq, lse, D of listed query rows (original token order) over their whole key set."""
        q_rows, dout_rows, k, v = _f32(q_rows), _f32(dout_rows), _f32(k), _f32(v)
        rb, rh, rt = (np.ascontiguousarray(x, np.int64) for x in (row_b, row_h, row_t))
        nrows, d = q_rows.shape
        _, Hkv, S, _ = k.shape
        dq = np.empty((nrows, d), np.float64)
        lse = np.empty(nrows, np.float64)
        Dv = np.empty(nrows, np.float64)
        self.lib.ora_bwd_query_rows(_ptr(q_rows), _ptr(dout_rows), _ptr(rb), _ptr(rh), _ptr(rt),
                                    nrows, _ptr(k), _ptr(v), Hq, Hkv, S, d, float(scale),
                                    int(bool(causal)), _ptr(dq), _ptr(lse), _ptr(Dv))
        return dq, lse, Dv

    def bwd_keys(self, q_rows, dout_rows, row_b, row_h, row_t, lse, Dv, key_b, key_g, key_t, k,
                 v, Hq: int, scale: float, causal: bool):
        """dk, dv of listed keys from the listed query rows (with their lse, D)."""
        q_rows, dout_rows, k, v = _f32(q_rows), _f32(dout_rows), _f32(k), _f32(v)
        rb, rh, rt, kb_, kg_, kt_ = (np.ascontiguousarray(x, np.int64)
                                     for x in (row_b, row_h, row_t, key_b, key_g, key_t))
        lse = np.ascontiguousarray(lse, np.float64)
        Dv = np.ascontiguousarray(Dv, np.float64)
        nrows, d = q_rows.shape
        _, Hkv, S, _ = k.shape
        dk = np.empty((len(kt_), d), np.float64)
        dv = np.empty((len(kt_), d), np.float64)
        self.lib.ora_bwd_keys(_ptr(q_rows), _ptr(dout_rows), _ptr(rb), _ptr(rh), _ptr(rt),
                              _ptr(lse), _ptr(Dv), nrows, _ptr(kb_), _ptr(kg_), _ptr(kt_),
                              len(kt_), _ptr(k), _ptr(v), Hq, Hkv, S, d, float(scale),
                              int(bool(causal)), _ptr(dk), _ptr(dv))
        return dk, dv

    def block_bwd(self, q, k, v, dout, lse, Dv, scale: float, causal: bool, qid, kid):
        """One (query shard, key block) pair's gradient contributions, given the
        global lse and D = <dO, O> per row: q, dout [B][Hq][nq][d]; k, v
        [B][Hkv][nk][d]; lse, Dv [B][Hq][nq]; qid [nq], kid [nk] global tokens."""
        q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
        lse = np.ascontiguousarray(lse, np.float64)
        Dv = np.ascontiguousarray(Dv, np.float64)
        qid = np.ascontiguousarray(qid, np.int64)
        kid = np.ascontiguousarray(kid, np.int64)
        B, Hq, nq, d = q.shape
        _, Hkv, nk, _ = k.shape
        dq = np.empty((B, Hq, nq, d), np.float64)
        dk = np.empty((B, Hkv, nk, d), np.float64)
        dv = np.empty((B, Hkv, nk, d), np.float64)
        self.lib.ora_block_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(Dv), B, Hq,
                               Hkv, nq, nk, d, float(scale), int(bool(causal)), _ptr(qid),
                               _ptr(kid), _ptr(dq), _ptr(dk), _ptr(dv))
        return dq, dk, dv


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c as committed (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def compile_variant(source_text: str, out_path: str) -> Oracle:
    """Compile a modified copy of oracle.c (used by tests that plant mistakes)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc"] + _CFLAGS + [src, "-o", out_path, "-lm"], check=True)
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def num_threads() -> int:
    return default().num_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def layout_maps(layout, S, R):
    return default().layout_maps(layout, S, R)


def attention_rows(*a, **kw):
    return default().attention_rows(*a, **kw)


def attention_full(*a, **kw):
    return default().attention_full(*a, **kw)


def attention_bwd(*a, **kw):
    return default().attention_bwd(*a, **kw)


def block_bwd(*a, **kw):
    return default().block_bwd(*a, **kw)


def bwd_query_rows(*a, **kw):
    return default().bwd_query_rows(*a, **kw)


def bwd_keys(*a, **kw):
    return default().bwd_keys(*a, **kw)


def block_partial(*a, **kw):
    return default().block_partial(*a, **kw)


def merge(*a, **kw):
    return default().merge(*a, **kw)


def ring_emulate(*a, **kw):
    return default().ring_emulate(*a, **kw)


def pair_counts(layout, S, R):
    return default().pair_counts(layout, S, R)
