"""Workload shapes for the pooled-wave MoE dispatch share.

Plain data only: sizes, capacity factors as exact rationals, and the kind of
routing skew each workload carries.  No part of the method is computed here.

Model constants (384 routed experts, top-8, 2 shared experts, width 6144,
latent 3072, a 64-GPU expert-parallel domain with 6 experts per GPU, three
waves, sender/receiver capacity factors 1.10/1.15) come from
"Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二,
and its Japanese translation "Marin、535BパラメータMoEモデルのオープン
トレーニングを開始" (lamjinlab.com, ja), section 二.  The pages leave the
routed-expert FFN open; a SwiGLU with intermediate 1536 is used (the same for
the two shared experts).  The 4096- and 65536-token lengths follow the
context schedule in section 四 of the same pages.
"""
from dataclasses import dataclass, replace
from fractions import Fraction
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens per source shard
    d_model: int      # model width
    latent: int       # latent width carried through the exchange
    n_experts: int    # routed experts
    n_ranks: int      # ranks of the expert-parallel domain (logical here)
    top_k: int
    n_waves: int
    d_ff: int         # routed SwiGLU intermediate
    n_shared: int
    d_ff_shared: int  # shared SwiGLU intermediate
    cf_send: Optional[Fraction]   # None = ragged / dropless
    cf_recv: Optional[Fraction]
    routing: str = "plain"        # "plain" | "zipf" | "longctx"
    shards: int = 0               # number of source shards (0 = n_ranks)
    # "tokens": wave(t) = t / T_w, a pool per (destination, wave); "chunks": one
    # pool of n_waves * C_s rows per destination, cut into n_waves chunks
    waves: str = "tokens"
    # variant: a token's choices on one destination share one row (up to 4 ids)
    dedup: bool = False

    @property
    def experts_per_rank(self) -> int:
        return self.n_experts // self.n_ranks

    @property
    def n_shards(self) -> int:
        return self.shards or self.n_ranks

    @property
    def ragged(self) -> bool:
        return self.cf_send is None


F110 = Fraction(110, 100)
F115 = Fraction(115, 100)

TINY = Workload("moe_tiny_T64_D256_L128_E48_R8", 64, 256, 128, 48, 8, 8, 3,
                256, 2, 256, F110, F115)
SHARE_4K = Workload("moe_share_T4096_D6144_L3072_E384_R64", 4096, 6144, 3072,
                    384, 64, 8, 3, 1536, 2, 1536, F110, F115)
ZIPF_16K = replace(SHARE_4K, name="moe_zipf_T16384_D6144_L3072_E384_R64",
                   T=16384, routing="zipf")
LONG_65K = replace(SHARE_4K, name="moe_longctx_T65536_D6144_L3072_E384_R64",
                   T=65536, routing="longctx")
SWEEP_16K = {
    "1.10/1.15": ZIPF_16K,
    "1.5/1.5": replace(ZIPF_16K, name=ZIPF_16K.name + "_cf1.5",
                       cf_send=Fraction(3, 2), cf_recv=Fraction(3, 2)),
    "2.0/2.0": replace(ZIPF_16K, name=ZIPF_16K.name + "_cf2.0",
                       cf_send=Fraction(2), cf_recv=Fraction(2)),
    "inf": replace(ZIPF_16K, name=ZIPF_16K.name + "_ragged",
                   cf_send=None, cf_recv=None),
}

# Index order of the five workloads.
WORKLOADS = [TINY, SHARE_4K, ZIPF_16K, LONG_65K, SWEEP_16K["inf"]]


def scaled(base: Workload, name: str, **kw) -> Workload:
    """A workload with some sizes changed (parity cases between tiny and full)."""
    return replace(base, name=name, **kw)
