"""Workload shapes of the routed MoE layer forward.

Sizes follow the pages' models: the 535B-A23B layer (Marin 535B-A23B article,
section "What is actually being trained"; launch blog section 2 "How the Sparse
Model Is Organized"), the 67B-A2B "Grug" shape, a tiny float32 case, one GPU's
expert-parallel share of the 535B layer (six local experts fed from a fixed
receiver pool, launch blog section 2), and a 65,536-token long-context batch with
skewed routing (launch blog section 4, "Long Context Depends on Solving Token
Dropping").
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    D: int          # model width
    L: int          # latent width (0: no latent; routing and experts act on x)
    E: int          # routed experts
    k: int          # experts per token
    H: int          # routed expert SwiGLU hidden width
    n_shared: int   # shared experts
    Hs: int         # shared expert hidden width
    dtype: str      # "f32" or "bf16": storage of activations and weights
    seed: int
    eps: float = 1e-5
    hot_frac: float = 0.0    # fraction of experts given a router bias
    hot_load: float = 1.0    # their target mean load relative to the mean

    @property
    def d_e(self) -> int:
        """Width the routed experts act on."""
        return self.L if self.L > 0 else self.D

    @property
    def R(self) -> int:
        """Routed rows when nothing is dropped."""
        return self.T * self.k

    def flops(self, kept_rows: int | None = None) -> int:
        """Model FLOPs of one forward: 2*M*N*K per matmul, the gated MLP counted as
        three matmuls, over kept rows only (router included, in float32)."""
        R = self.R if kept_rows is None else kept_rows
        T, D, L, de = self.T, self.D, self.L, self.d_e
        f = 0
        if L > 0:
            f += 2 * T * D * L * 2                      # down and up projections
        f += 2 * T * de * self.E                        # router logits
        f += 2 * R * de * self.H * 3                    # routed gate, up, down
        f += 2 * T * D * self.Hs * 3 * self.n_shared    # shared experts
        return f


@dataclass(frozen=True)
class PoolConfig:
    """One GPU's expert-parallel share: a fixed receiver pool of rows that senders
    filled, each row carrying its local expert id (-1 marks padding)."""
    name: str
    n_senders: int
    slot_rows: int        # rows per sender slot = ceil(1.10 * mu)
    mu: float             # expected rows per sender
    sigma: float          # log-normal spread of a sender's row count
    E: int                # local experts
    L: int                # latent width
    H: int                # expert hidden width
    zipf_s: float
    seed: int
    dtype: str = "bf16"

    @property
    def P(self) -> int:
        return self.n_senders * self.slot_rows

    def flops(self, valid_rows: int) -> int:
        return 2 * valid_rows * self.L * self.H * 3


@dataclass(frozen=True)
class ExpertMlpConfig:
    """Routed rows through the gated expert MLP, forward and backward: T tokens
    each routed to k distinct experts (uniformly at random, or Zipf(zipf_s) over
    the experts when k = 1), rows grouped by expert."""
    name: str
    T: int
    d: int          # width the experts act on
    H: int          # expert hidden width
    E: int
    k: int
    seed: int
    zipf_s: float = 0.0
    dtype: str = "bf16"

    @property
    def R(self) -> int:
        return self.T * self.k

    def flops_fwd(self) -> int:
        return 2 * self.R * self.d * self.H * 3          # gate, up, down

    def flops_bwd(self) -> int:
        # dh, dW_d, dX, dW_gu (the last two over 2H): six matmuls of the forward's size
        return 2 * self.R * self.d * self.H * 6


TINY = LayerConfig("tiny_f32_T256_D256_L128_E16_k2", T=256, D=256, L=128, E=16, k=2, H=128,
                   n_shared=1, Hs=128, dtype="f32", seed=0)
GRUG67B = LayerConfig("grug67b_bf16_T8192_D2048_E64_k4", T=8192, D=2048, L=0, E=64, k=4,
                      H=1024, n_shared=1, Hs=2048, dtype="bf16", seed=1)
MARIN535B = LayerConfig("marin535b_bf16_T8192_D6144_L3072_E384_k8", T=8192, D=6144, L=3072,
                        E=384, k=8, H=3072, n_shared=2, Hs=3072, dtype="bf16", seed=2)
EP_SHARE = PoolConfig("marin535b_ep_share_bf16_P65536_E6", n_senders=64, slot_rows=1024,
                      mu=1024 / 1.10, sigma=0.17, E=6, L=3072, H=3072, zipf_s=1.0, seed=3)
LONGCTX = LayerConfig("marin535b_longctx_bf16_T65536_D6144_L3072_E384_k8", T=65536, D=6144,
                      L=3072, E=384, k=8, H=3072, n_shared=2, Hs=3072, dtype="bf16", seed=4,
                      hot_frac=0.10, hot_load=5.0)

# The pages' custom-VJP microbench of the Grug MoE expert MLP (Marin: Week of
# April 26th summary, the paragraph on moving the backward pass onto Triton):
# 4,096 tokens, hidden 1,024, intermediate 2,048, 64 experts, top-4, bf16.
GRUG_VJP = ExpertMlpConfig("grug_vjp_bf16_T4096_D1024_H2048_E64_k4", T=4096, d=1024, H=2048,
                           E=64, k=4, seed=6)
# The 535B layer's routed rows (8,192 tokens x top-8 of 384 experts on the latent)
# and one GPU's receiver pool of six local experts.
MARIN535B_EXPERTS = ExpertMlpConfig("marin535b_experts_bf16_T8192_L3072_H3072_E384_k8", T=8192,
                                    d=3072, H=3072, E=384, k=8, seed=7)
EP_SHARE_EXPERTS = ExpertMlpConfig("marin535b_ep_share_experts_bf16_R61440_E6", T=61440, d=3072,
                                   H=3072, E=6, k=1, seed=8, zipf_s=1.0)

CONFIGS = [TINY, GRUG67B, MARIN535B, EP_SHARE, LONGCTX]
MLP_CONFIGS = [GRUG_VJP, MARIN535B_EXPERTS, EP_SHARE_EXPERTS]


def by_name(name: str):
    for c in CONFIGS + MLP_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
