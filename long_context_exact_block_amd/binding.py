"""ctypes binding of libra.so (the C ABI declared in include/ra.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libra.so.  PyTorch tensors provide device memory and streams.
If the library is missing the calls raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# RA_LIBRARY names another build of the same library (the tests' host-only
# sanitizer build); by default the in-tree libra.so
LIB_PATH = os.environ.get("RA_LIBRARY") or os.path.join(PKG, "libra.so")

RA_OK = 0
STATUS_NAMES = {0: "RA_OK", 1: "RA_ERR_INVALID_ARG", 2: "RA_ERR_SHAPE", 3: "RA_ERR_DTYPE",
                4: "RA_ERR_ALIGNMENT", 5: "RA_ERR_WORKSPACE", 6: "RA_ERR_UNSUPPORTED",
                7: "RA_ERR_HIP"}
LAYOUT_CONTIGUOUS, LAYOUT_STRIPED, LAYOUT_ZIGZAG = 0, 1, 2
DT_BF16, DT_FP16, DT_FP32 = 0, 1, 2
HANDOFF_COPY, HANDOFF_SWAP, HANDOFF_FORWARD = 0, 1, 2
MERGE_FUSED, MERGE_SEPARATE = 0, 1

LAYOUTS = {"contiguous": LAYOUT_CONTIGUOUS, "striped": LAYOUT_STRIPED, "zigzag": LAYOUT_ZIGZAG}

EXPORTED = ("ra_version", "ra_status_string", "ra_last_error", "ra_layout_permute",
            "ra_layout_gather", "ra_layout_scatter", "ra_block_fwd", "ra_packed_v_bytes",
            "ra_pack_v", "ra_merge", "ra_finalize", "ra_ring_fwd_workspace_size", "ra_ring_fwd",
            "ra_causal_work", "ra_decode_fwd_workspace_size", "ra_decode_fwd",
            "ra_block_bwd_workspace_size", "ra_block_bwd", "ra_ring_bwd_workspace_size",
            "ra_ring_bwd", "ra_handoff_copy", "ra_handoff_thin", "ra_decode_fwd_noalloc",
            "ra_cached_events")


class RAError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__("%s: %s" % (self.name, detail))


I64 = ctypes.c_int64
I32 = ctypes.c_int32
P = ctypes.c_void_p


class BlockArgs(ctypes.Structure):
    _fields_ = [("q", P), ("k", P), ("v", P), ("dtype", I32), ("v_packed", I32), ("B", I32),
                ("Hq", I32),
                ("Hkv", I32), ("n_q", I32), ("n_k", I32), ("d", I32), ("q_stride", I64 * 3),
                ("k_stride", I64 * 3), ("v_stride", I64 * 3), ("scale", ctypes.c_float),
                ("causal", I32), ("q_gid0", I64), ("q_gid_step", I64), ("k_gid0", I64),
                ("k_gid_step", I64), ("o", P), ("o_stride", I64 * 3), ("m", P), ("l", P)]


class RingArgs(ctypes.Structure):
    _fields_ = [("q_sh", P), ("k_sh", P), ("v_sh", P), ("dtype", I32), ("R", I32),
                ("rank0", I32), ("n_ranks", I32), ("B", I32), ("Hq", I32), ("Hkv", I32),
                ("n", I32), ("d", I32), ("scale", ctypes.c_float), ("causal", I32),
                ("layout", I32), ("handoff", I32), ("merge_mode", I32), ("o", P), ("lse", P),
                ("hop_events", ctypes.POINTER(P))]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", P), ("k", P), ("v", P), ("dtype", I32), ("R", I32), ("B", I32),
                ("Hq", I32), ("Hkv", I32), ("nq", I32), ("n", I32), ("d", I32),
                ("scale", ctypes.c_float), ("causal", I32), ("q_gid0", I64), ("o", P), ("lse", P)]


class BlockBwdArgs(ctypes.Structure):
    _fields_ = [("q", P), ("k", P), ("v", P), ("o", P), ("dout", P), ("dtype", I32), ("B", I32),
                ("Hq", I32), ("Hkv", I32), ("n_q", I32), ("n_k", I32), ("d", I32),
                ("scale", ctypes.c_float), ("causal", I32), ("q_gid0", I64), ("q_gid_step", I64),
                ("k_gid0", I64), ("k_gid_step", I64), ("lse", P), ("dq", P), ("dk", P), ("dv", P)]


class RingBwdArgs(ctypes.Structure):
    _fields_ = [("q_sh", P), ("k_sh", P), ("v_sh", P), ("o_sh", P), ("dout_sh", P), ("lse", P),
                ("dtype", I32), ("R", I32), ("rank0", I32), ("n_ranks", I32), ("B", I32),
                ("Hq", I32), ("Hkv", I32), ("n", I32), ("d", I32), ("scale", ctypes.c_float),
                ("causal", I32), ("layout", I32), ("handoff", I32), ("dq_sh", P), ("dk_sh", P),
                ("dv_sh", P)]


_lib = None


def lib():
    """Load libra.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libra.so is not built (run __graft_entry__.build() or "
                           "python -m long_context_exact_block_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.ra_version.restype = ctypes.c_int
    L.ra_status_string.restype = ctypes.c_char_p
    L.ra_status_string.argtypes = [ctypes.c_int]
    L.ra_last_error.restype = ctypes.c_char_p
    L.ra_layout_permute.argtypes = [I32, I64, I32, P, P, P]
    L.ra_layout_gather.argtypes = [P, P, P, I32, I64, I64, I64, I64, I32, I32, I32, P]
    L.ra_layout_scatter.argtypes = [P, P, P, I32, I64, I64, I64, I64, I32, I32, I32, P]
    L.ra_block_fwd.argtypes = [ctypes.POINTER(BlockArgs), P]
    L.ra_block_bwd_workspace_size.argtypes = [ctypes.POINTER(BlockBwdArgs)]
    L.ra_block_bwd_workspace_size.restype = ctypes.c_size_t
    L.ra_block_bwd.argtypes = [ctypes.POINTER(BlockBwdArgs), P, ctypes.c_size_t, P]
    L.ra_ring_bwd_workspace_size.argtypes = [ctypes.POINTER(RingBwdArgs)]
    L.ra_ring_bwd_workspace_size.restype = ctypes.c_size_t
    L.ra_ring_bwd.argtypes = [ctypes.POINTER(RingBwdArgs), P, ctypes.c_size_t, P, P]
    L.ra_decode_fwd_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs)]
    L.ra_decode_fwd_workspace_size.restype = ctypes.c_size_t
    L.ra_decode_fwd.argtypes = [ctypes.POINTER(DecodeArgs), P, ctypes.c_size_t, P]
    L.ra_decode_fwd_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), P]
    L.ra_cached_events.restype = ctypes.c_size_t
    L.ra_packed_v_bytes.argtypes = [I32, I32, I32, I32, I32]
    L.ra_packed_v_bytes.restype = ctypes.c_size_t
    L.ra_pack_v.argtypes = [P, P, I32, I32, I32, I32, I32, ctypes.POINTER(I64), P]
    L.ra_handoff_copy.argtypes = [P, P, ctypes.c_size_t, I32, P]
    L.ra_handoff_thin.argtypes = [ctypes.c_double, ctypes.c_double, I32, ctypes.c_double]
    L.ra_handoff_thin.restype = I32
    L.ra_merge.argtypes = [P, P, P, P, P, P, I64, I32, P]
    L.ra_finalize.argtypes = [P, P, P, P, P, I32, I64, I32, P]
    L.ra_ring_fwd_workspace_size.argtypes = [ctypes.POINTER(RingArgs)]
    L.ra_ring_fwd_workspace_size.restype = ctypes.c_size_t
    L.ra_ring_fwd.argtypes = [ctypes.POINTER(RingArgs), P, ctypes.c_size_t, P, P]
    L.ra_causal_work.argtypes = [I32, I64, I32, P]
    for name in ("ra_layout_permute", "ra_layout_gather", "ra_layout_scatter", "ra_block_fwd",
                 "ra_pack_v", "ra_merge", "ra_finalize", "ra_ring_fwd", "ra_causal_work"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status):
    if status != RA_OK:
        raise RAError(status, lib().ra_last_error().decode())


def last_error() -> str:
    return lib().ra_last_error().decode()


# --------------------------------------------------------------------------- torch helpers
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    torch = _torch()
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t) -> int:
    torch = _torch()
    return {torch.bfloat16: DT_BF16, torch.float16: DT_FP16, torch.float32: DT_FP32}[t.dtype]


# --------------------------------------------------------------------------- entry points
def ra_layout_permute(layout: int, S: int, R: int, fwd, inv=None, stream=None):
    _check(lib().ra_layout_permute(int(layout), int(S), int(R), _ptr(fwd), _ptr(inv),
                                   _stream(stream)))


def ra_layout_gather(x, x_sh, fwd, R: int, rank0: int = 0, n_ranks: int = -1, stream=None):
    """x [B][H][S][d] -> x_sh [n_ranks][B][H][S/R][d]."""
    B, H, S, d = x.shape
    n_ranks = R if n_ranks < 0 else n_ranks
    _check(lib().ra_layout_gather(_ptr(x), _ptr(x_sh), _ptr(fwd), x.element_size(), B, H, S, d,
                                  int(R), int(rank0), int(n_ranks), _stream(stream)))


def ra_layout_scatter(x_sh, x, fwd, R: int, rank0: int = 0, n_ranks: int = -1, stream=None):
    """x_sh [n_ranks][B][H][S/R][d] -> rows of x [B][H][S][d] owned by those ranks."""
    B, H, S, d = x.shape
    n_ranks = R if n_ranks < 0 else n_ranks
    _check(lib().ra_layout_scatter(_ptr(x_sh), _ptr(x), _ptr(fwd), x.element_size(), B, H, S, d,
                                   int(R), int(rank0), int(n_ranks), _stream(stream)))


def block_args(q, k, v, o, m, l, scale, causal, q_gid0=0, q_gid_step=1, k_gid0=0,
               k_gid_step=1, v_packed=False) -> BlockArgs:
    B, Hq, nq, d = q.shape
    _, Hkv, nk, _ = k.shape
    a = BlockArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.dtype = dtype_code(q)
    a.v_packed = int(bool(v_packed))
    a.B, a.Hq, a.Hkv, a.n_q, a.n_k, a.d = B, Hq, Hkv, nq, nk, d
    for i in range(3):
        a.q_stride[i] = q.stride(i)
        a.k_stride[i] = k.stride(i)
        a.v_stride[i] = 0 if v_packed else v.stride(i)
        a.o_stride[i] = o.stride(i)
    a.scale = float(scale)
    a.causal = int(bool(causal))
    a.q_gid0, a.q_gid_step, a.k_gid0, a.k_gid_step = q_gid0, q_gid_step, k_gid0, k_gid_step
    a.o, a.m, a.l = o.data_ptr(), m.data_ptr(), l.data_ptr()
    return a


def ra_block_fwd(q, k, v, o, m, l, scale, causal, q_gid0=0, q_gid_step=1, k_gid0=0,
                 k_gid_step=1, stream=None, v_packed=False):
    """q [B][Hq][nq][d], k, v [B][Hkv][nk][d] -> o fp32 [B][Hq][nq][d], m, l fp32 [B][Hq][nq].

    With v_packed=True, v is the buffer ra_pack_v filled for this K/V block."""
    a = block_args(q, k, v, o, m, l, scale, causal, q_gid0, q_gid_step, k_gid0, k_gid_step,
                   v_packed)
    _check(lib().ra_block_fwd(ctypes.byref(a), _stream(stream)))


def ra_packed_v_bytes(dtype: int, B: int, H: int, n: int, d: int) -> int:
    nb = lib().ra_packed_v_bytes(int(dtype), int(B), int(H), int(n), int(d))
    if nb == 0 and last_error():
        raise RAError(3, last_error())
    return int(nb)


def ra_pack_v(v, vp, stream=None):
    """v [B][H][n][d] (bf16/fp16, strided rows) -> vp (uint8/16-bit buffer of
    ra_packed_v_bytes bytes) in the packed layout."""
    B, H, n, d = v.shape
    st = (I64 * 3)(v.stride(0), v.stride(1), v.stride(2))
    _check(lib().ra_pack_v(_ptr(v), _ptr(vp), dtype_code(v), B, H, n, d, st, _stream(stream)))


def ra_handoff_copy(dst, src, nbytes=None, stream=None, thin=False):
    """Device copy of nbytes (default: all of src) from src to dst, as the ring's hand-off
    (thin: the one-wave form the rings use for long hops)."""
    nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().ra_handoff_copy(_ptr(dst), _ptr(src), nb, int(bool(thin)), _stream(stream)))


def thin_handoff(moved_bytes, pairs_heads, d, work=1.0):
    """Whether a ring uses the thin hand-off copy (the library's rule, ra_handoff_thin)."""
    return bool(lib().ra_handoff_thin(float(moved_bytes), float(pairs_heads), int(d), float(work)))


def ra_merge(o_acc, m_acc, l_acc, o_blk, m_blk, l_blk, stream=None):
    rows = m_acc.numel()
    d = o_acc.numel() // max(rows, 1)
    _check(lib().ra_merge(_ptr(o_acc), _ptr(m_acc), _ptr(l_acc), _ptr(o_blk), _ptr(m_blk),
                          _ptr(l_blk), rows, d, _stream(stream)))


def ra_finalize(o_acc, m, l, out, lse, stream=None):
    rows = m.numel()
    d = o_acc.numel() // max(rows, 1)
    _check(lib().ra_finalize(_ptr(o_acc), _ptr(m), _ptr(l), _ptr(out), _ptr(lse),
                             dtype_code(out), rows, d, _stream(stream)))


def ring_args(q_sh, k_sh, v_sh, o, lse, R, rank0, n_ranks, scale, causal, layout,
              handoff=HANDOFF_COPY, merge_mode=MERGE_FUSED) -> RingArgs:
    _, B, Hq, n, d = q_sh.shape
    Hkv = k_sh.shape[2]
    a = RingArgs()
    a.q_sh, a.k_sh, a.v_sh = q_sh.data_ptr(), k_sh.data_ptr(), v_sh.data_ptr()
    a.dtype = dtype_code(q_sh)
    a.R, a.rank0, a.n_ranks = int(R), int(rank0), int(n_ranks)
    a.B, a.Hq, a.Hkv, a.n, a.d = B, Hq, Hkv, n, d
    a.scale = float(scale)
    a.causal = int(bool(causal))
    a.layout = int(layout)
    a.handoff = int(handoff)
    a.merge_mode = int(merge_mode)
    a.o = o.data_ptr()
    a.lse = lse.data_ptr()
    return a


def ra_ring_fwd_workspace_size(args: RingArgs) -> int:
    n = lib().ra_ring_fwd_workspace_size(ctypes.byref(args))
    if n == 0:
        err = last_error()
        if err:
            raise RAError(2, err)
    return int(n)


def ra_ring_fwd(args: RingArgs, workspace, compute_stream=None, copy_stream=None):
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().ra_ring_fwd(ctypes.byref(args), ws_ptr, ws_bytes, cs, xs))


def block_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, q_gid0=0, q_step=1,
                   k_gid0=0, k_step=1) -> BlockBwdArgs:
    """q, o, dout [B][Hq][nq][d]; k, v [B][Hkv][nk][d] (16-bit, contiguous); lse fp32
    [B][Hq][nq]; dq, dk, dv fp32 accumulators shaped like q, k, v."""
    B, Hq, nq, d = q.shape
    _, Hkv, nk, _ = k.shape
    a = BlockBwdArgs()
    a.q, a.k, a.v, a.o, a.dout = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout)
    a.dtype = dtype_code(q)
    a.B, a.Hq, a.Hkv, a.n_q, a.n_k, a.d = B, Hq, Hkv, nq, nk, d
    a.scale, a.causal = float(scale), int(bool(causal))
    a.q_gid0, a.q_gid_step, a.k_gid0, a.k_gid_step = int(q_gid0), int(q_step), int(k_gid0), int(k_step)
    a.lse, a.dq, a.dk, a.dv = _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv)
    return a


def ra_block_bwd_workspace_size(args: BlockBwdArgs) -> int:
    nb = lib().ra_block_bwd_workspace_size(ctypes.byref(args))
    if nb == 0 and args.n_q > 0:
        raise RAError(1, last_error())
    return nb


def ra_block_bwd(args: BlockBwdArgs, workspace, stream=None):
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().ra_block_bwd(ctypes.byref(args), ws_ptr, ws_bytes, _stream(stream)))


def ring_bwd_args(q_sh, k_sh, v_sh, o_sh, dout_sh, lse, dq_sh, dk_sh, dv_sh, R, rank0, n_ranks,
                  scale, causal, layout, handoff=HANDOFF_COPY) -> RingBwdArgs:
    """Shards as for ra_ring_fwd: q_sh, o_sh, dout_sh, dq_sh [n_ranks][B][Hq][n][d];
    k_sh, v_sh, dk_sh, dv_sh [R][B][Hkv][n][d]; lse fp32 [n_ranks][B][Hq][n]."""
    _, B, Hq, n, d = q_sh.shape
    Hkv = k_sh.shape[2]
    a = RingBwdArgs()
    a.q_sh, a.k_sh, a.v_sh, a.o_sh, a.dout_sh = (_ptr(x) for x in (q_sh, k_sh, v_sh, o_sh, dout_sh))
    a.lse = _ptr(lse)
    a.dtype = dtype_code(q_sh)
    a.R, a.rank0, a.n_ranks = R, rank0, n_ranks
    a.B, a.Hq, a.Hkv, a.n, a.d = B, Hq, Hkv, n, d
    a.scale, a.causal = float(scale), int(bool(causal))
    a.layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    a.handoff = int(handoff)
    a.dq_sh, a.dk_sh, a.dv_sh = _ptr(dq_sh), _ptr(dk_sh), _ptr(dv_sh)
    return a


def ra_ring_bwd_workspace_size(args: RingBwdArgs) -> int:
    nb = lib().ra_ring_bwd_workspace_size(ctypes.byref(args))
    if nb == 0 and args.n > 0:
        raise RAError(1, last_error())
    return nb


def ra_ring_bwd(args: RingBwdArgs, workspace, compute_stream=None, copy_stream=None):
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().ra_ring_bwd(ctypes.byref(args), ws_ptr, ws_bytes, cs, xs))


def decode_args(q, k, vp, o, lse, scale, causal, q_gid0) -> DecodeArgs:
    """q [B][Hq][nq][d]; k [R][B][Hkv][n][d]; vp: ra_pack_v of V as [R*B][Hkv][n][d];
    o like q; lse fp32 [B][Hq][nq]."""
    B, Hq, nq, d = q.shape
    R, _, Hkv, n, _ = k.shape
    a = DecodeArgs()
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(vp)
    a.dtype = dtype_code(q)
    a.R, a.B, a.Hq, a.Hkv, a.nq, a.n, a.d = R, B, Hq, Hkv, nq, n, d
    a.scale, a.causal, a.q_gid0 = float(scale), int(bool(causal)), int(q_gid0)
    a.o, a.lse = _ptr(o), _ptr(lse)
    return a


def ra_decode_fwd_workspace_size(args: DecodeArgs) -> int:
    nb = lib().ra_decode_fwd_workspace_size(ctypes.byref(args))
    if nb == 0:
        raise RAError(1, last_error())
    return nb


def ra_decode_fwd(args: DecodeArgs, workspace, stream=None):
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().ra_decode_fwd(ctypes.byref(args), ws_ptr, ws_bytes, _stream(stream)))


def ra_decode_fwd_noalloc(args: DecodeArgs, stream=None):
    """ra_decode_fwd with the partials in the library's per-GPU device array (no workspace)."""
    _check(lib().ra_decode_fwd_noalloc(ctypes.byref(args), _stream(stream)))


def ra_causal_work(layout: int, S: int, R: int):
    import numpy as np
    W = np.zeros(R, np.int64)
    _check(lib().ra_causal_work(int(layout), int(S), int(R),
                                W.ctypes.data_as(ctypes.c_void_p)))
    return W


def ra_cached_events() -> int:
    """Number of HIP events the library caches for its ring drivers (diagnostic)."""
    return int(lib().ra_cached_events())
