"""One pass of the whole ring-attention path on one GPU, from inputs in the
original token order to outputs in the original token order:

  index maps (ra_layout_permute) -> shard gather of Q, K, V (ra_layout_gather)
  -> R hops of block attention + online-softmax fold with the K/V hand-off (a
  copy on a side stream, or written on by the block kernel: ra_ring_fwd's
  COPY / FORWARD) -> scatter of O and LSE back (ra_layout_scatter).

Device memory and streams come from PyTorch; every step runs in libra.so.
"""
from __future__ import annotations

import math

from . import binding as rb


class RingAttention:
    """Buffers and streams for one workload shape; ``run`` performs one pass.

    q [B][Hq][S][d], k, v [B][Hkv][S][d] (bf16 / fp16 / fp32, original order).
    Computed query ranks are rank0 .. rank0+n_ranks-1 of R; only their rows of
    the output are written.
    """

    def __init__(self, B, Hq, Hkv, S, d, R, layout="striped", dtype=None, causal=True, scale=None,
                 rank0=0, n_ranks=-1, handoff=rb.HANDOFF_COPY, merge_mode=rb.MERGE_FUSED,
                 device="cuda", copy_stream=True):
        import torch
        if S % R:
            raise ValueError("S must be divisible by R")
        self.torch = torch
        self.B, self.Hq, self.Hkv, self.S, self.d, self.R = B, Hq, Hkv, S, d, R
        self.n = S // R
        self.layout = rb.LAYOUTS[layout] if isinstance(layout, str) else int(layout)
        self.dtype = dtype or torch.bfloat16
        self.causal = bool(causal)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.rank0 = rank0
        self.n_ranks = R if n_ranks < 0 else n_ranks
        self.handoff = handoff
        self.merge_mode = merge_mode
        dev = torch.device(device)
        n, nr = self.n, self.n_ranks
        self.fwd = torch.empty(S, dtype=torch.int32, device=dev)
        self.inv = torch.empty(S, dtype=torch.int32, device=dev)
        self.q_sh = torch.empty((nr, B, Hq, n, d), dtype=self.dtype, device=dev)
        self.k_sh = torch.empty((R, B, Hkv, n, d), dtype=self.dtype, device=dev)
        self.v_sh = torch.empty((R, B, Hkv, n, d), dtype=self.dtype, device=dev)
        self.o_sh = torch.empty((nr, B, Hq, n, d), dtype=self.dtype, device=dev)
        self.lse_sh = torch.empty((nr, B, Hq, n), dtype=torch.float32, device=dev)
        self.args = rb.ring_args(self.q_sh, self.k_sh, self.v_sh, self.o_sh, self.lse_sh, R,
                                 rank0, nr, self.scale, self.causal, self.layout, handoff,
                                 merge_mode)
        ws = rb.ra_ring_fwd_workspace_size(self.args)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.copy_stream = torch.cuda.Stream(device=dev) if copy_stream else None

    def maps(self, stream=None):
        rb.ra_layout_permute(self.layout, self.S, self.R, self.fwd, self.inv, stream)

    def gather(self, q, k, v, stream=None):
        rb.ra_layout_gather(q, self.q_sh, self.fwd, self.R, self.rank0, self.n_ranks, stream)
        rb.ra_layout_gather(k, self.k_sh, self.fwd, self.R, 0, self.R, stream)
        rb.ra_layout_gather(v, self.v_sh, self.fwd, self.R, 0, self.R, stream)

    def ring(self, stream=None):
        rb.ra_ring_fwd(self.args, self.workspace, stream, self.copy_stream)

    def scatter(self, o, lse, stream=None):
        rb.ra_layout_scatter(self.o_sh, o, self.fwd, self.R, self.rank0, self.n_ranks, stream)
        rb.ra_layout_scatter(self.lse_sh.unsqueeze(-1), lse.unsqueeze(-1), self.fwd, self.R,
                             self.rank0, self.n_ranks, stream)

    def run(self, q, k, v, o, lse, stream=None):
        """One full pass; o [B][Hq][S][d] (dtype), lse [B][Hq][S] fp32 (computed rows only)."""
        self.maps(stream)
        self.gather(q, k, v, stream)
        self.ring(stream)
        self.scatter(o, lse, stream)

    def backward(self, dout, dq, dk, dv, stream=None):
        """Gradients after ``run`` (same inputs still gathered): dout [B][Hq][S][d] in the
        original order; writes dq (rows of the computed ranks) and dk, dv [B][Hkv][S][d]
        (contributions of the computed ranks' queries), original order, in dtype."""
        torch = self.torch
        nr, R, n = self.n_ranks, self.R, self.n
        if not hasattr(self, "do_sh"):
            dev = self.q_sh.device
            self.do_sh = torch.empty_like(self.q_sh)
            self.dq_sh = torch.empty_like(self.q_sh)
            self.dk_sh = torch.empty_like(self.k_sh)
            self.dv_sh = torch.empty_like(self.v_sh)
            self.bargs = rb.ring_bwd_args(self.q_sh, self.k_sh, self.v_sh, self.o_sh, self.do_sh,
                                          self.lse_sh, self.dq_sh, self.dk_sh, self.dv_sh, R,
                                          self.rank0, nr, self.scale, self.causal, self.layout,
                                          self.handoff)
            nb = rb.ra_ring_bwd_workspace_size(self.bargs)
            self.bworkspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        rb.ra_layout_gather(dout, self.do_sh, self.fwd, R, self.rank0, nr, stream)
        rb.ra_ring_bwd(self.bargs, self.bworkspace, stream, self.copy_stream)
        rb.ra_layout_scatter(self.dq_sh, dq, self.fwd, R, self.rank0, nr, stream)
        rb.ra_layout_scatter(self.dk_sh, dk, self.fwd, R, 0, R, stream)
        rb.ra_layout_scatter(self.dv_sh, dv, self.fwd, R, 0, R, stream)
