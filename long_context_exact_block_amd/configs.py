"""The five workload shapes the ring attention path is tested and measured on.

Each is a synthetic stand-in for the pages' own framing (no page measures on a
dataset): a tiny fp32 case, the 32k-into-8x4k split of the SP/EP article, a
grouped-query case with a peaky softmax, one rank's share of a 1M-token
context over 8 ranks (the de/th Ring Attention guides' real-world example),
and 512-token shards (the SP/EP article's minimum sub-sequence).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    index: int           # 1-based workload number, also the seed family (1000*index)
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    R: int
    layouts: tuple       # ("striped",), ("contiguous", "striped"), ...
    causal: bool
    dtype: str           # "fp32" | "bf16" | "fp16"
    q_scale: float = 1.0
    rank0: int = 0       # first computed query rank
    n_ranks: int = -1    # number of computed query ranks (-1: all R)
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return self.S // self.R

    @property
    def ranks(self) -> int:
        return self.R if self.n_ranks < 0 else self.n_ranks

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 * self.index

    def metric_flops(self) -> float:
        """4*B*H*Sq*Sk*d, halved when causal (H = query heads)."""
        sq = self.n * self.ranks
        f = 4.0 * self.B * self.Hq * sq * self.S * self.d
        return f / 2 if self.causal else f


TINY = Workload("tiny_causal_fp32_S1k_R4", 1, 1, 2, 2, 64, 1024, 4, ("striped",), True, "fp32")
MHA_32K = Workload("causal_mha_bf16_S32k_R8", 2, 1, 32, 32, 128, 32768, 8,
                   ("contiguous", "striped"), True, "bf16")
GQA_128K = Workload("causal_gqa_bf16_S128k_R8_peaky", 3, 1, 32, 8, 128, 131072, 8, ("striped",),
                    True, "bf16", q_scale=4.0)
SHARE_1M = Workload("rank3_of_8_share_1M_striped_bf16", 4, 1, 8, 8, 128, 1048576, 8, ("striped",),
                    True, "bf16", rank0=3, n_ranks=1)
SHORT_512 = Workload("noncausal_fp16_S32k_R64_512tok", 5, 4, 16, 16, 64, 32768, 64,
                     ("contiguous",), False, "fp16")

ALL = (TINY, MHA_32K, GQA_128K, SHARE_1M, SHORT_512)
BY_NAME = {w.name: w for w in ALL}


@dataclass(frozen=True)
class DecodeWorkload:
    """nq new query tokens against a KV cache of S tokens split contiguously over R ranks."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    R: int
    nq: int
    causal: bool
    dtype: str
    seed: int

    @property
    def n(self) -> int:
        return self.S // self.R

    def cache_bytes(self) -> int:
        """K and V of the whole cache in the input dtype (each key read once)."""
        elt = 4 if self.dtype == "fp32" else 2
        return 2 * self.B * self.Hkv * self.S * self.d * elt

    def io_bytes(self) -> int:
        """Algorithmic bytes of one decode step: the cache, the new queries, O and LSE."""
        elt = 4 if self.dtype == "fp32" else 2
        rows = self.B * self.Hq * self.nq
        return self.cache_bytes() + rows * self.d * elt * 2 + rows * 4


# the long-context decode step: 4 new tokens (e.g. speculative decoding) against a
# 1M-token cache sharded over 8 ranks, grouped heads 32 -> 8, bf16
DECODE_1M = DecodeWorkload("decode_4tok_gqa_bf16_cache1M_R8", 1, 32, 8, 128, 1048576, 8, 4, True,
                           "bf16", 6000)
