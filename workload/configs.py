"""Shapes of the synthetic workloads.

Every workload is one expert-parallel (EP) layer as described on the Marin
535B-A23B pages ("Marin 开始公开训练 535B 参数 MoE 模型", lamjinlab blog,
section 二 "稀疏模型如何组织"): a 6144-wide model state, a router choosing 8 of
384 routed experts, a 3072-wide latent exchanged between GPUs, a 64-GPU EP
domain with 6 routed experts per GPU, a send capacity factor of 1.10, a
receive capacity factor of 1.15, three equal-shape waves and 2 always-on
shared experts.  The expert hidden widths (1536) and the activation (SwiGLU)
are not fixed by the pages; they are the widths of the one-rank layer this
package measures.

This module holds shapes only.  Capacities are derived elsewhere (the oracle
and the C library compute them independently).
"""

from dataclasses import dataclass, replace, asdict


@dataclass(frozen=True)
class Shape:
    name: str
    tokens: int            # T: tokens owned by one rank
    d_model: int           # D
    latent: int            # L
    n_experts: int         # E (routed)
    top_k: int             # k
    n_ranks: int           # R: EP domain size
    waves: int             # W: waves on the receive side
    expert_hidden: int     # H: routed expert SwiGLU hidden width
    shared_experts: int    # S
    shared_hidden: int     # HS
    act: str               # "bf16" or "f32": storage type of activations/weights
    send_num: int = 110    # send capacity factor 1.10 as a rational
    send_den: int = 100
    recv_num: int = 115    # receive capacity factor 1.15 as a rational
    recv_den: int = 100
    # workload structure
    emulate_all_ranks: bool = False   # True: every rank's tokens are generated
    bias: str = "none"                # "none" | "zipf" | "segments"
    segment_tokens: int = 512         # for bias == "segments"
    segment_hot: int = 16             # experts boosted per segment
    segment_boost: float = 3.0        # logit boost of a segment's hot experts
    zipf_s: float = 1.1
    zipf_std: float = 2.0
    receiver: str = "rank0"           # "rank0" | "hot_expert" (host of argmax bias)
    layer: str = "full"               # "dispatch" (route+pack) | "full"
    # one-rank workloads: how the other ranks' pools to the measured rank arise
    #   "routed": every other rank's own seeded tokens go through the same router
    #   "drawn":  pool contents drawn from a model of the arrivals (see gen.py)
    foreign: str = "routed"

    @property
    def local_experts(self):
        return self.n_experts // self.n_ranks

    def as_dict(self):
        return asdict(self)


# The five workloads of the one-rank layer.  1: tiny fp32, all 4 ranks
# emulated.  2: dispatch only at the production routing shape.  3: the full
# one-rank layer at 4K context (8192 tokens = 2 sequences of 4096).  4: the
# dispatch shape with a Zipf(1.1) per-expert router bias scaled to std 2.
# 5: one 65536-token sequence per rank with routing correlated inside
# 512-token segments.  6: config 3 with the wider experts (hidden 3072).  In 2-4 the other 63 ranks' tokens go through the same
# router; in 5 (64 x 65536 tokens would be 52 GB) their pools are drawn.
CONFIGS = {
    1: Shape("cfg1_tiny_f32", tokens=256, d_model=64, latent=32, n_experts=24,
             top_k=2, n_ranks=4, waves=3, expert_hidden=64, shared_experts=1,
             shared_hidden=64, act="f32", emulate_all_ranks=True),
    2: Shape("cfg2_dispatch_4k", tokens=8192, d_model=6144, latent=3072,
             n_experts=384, top_k=8, n_ranks=64, waves=3, expert_hidden=1536,
             shared_experts=2, shared_hidden=1536, act="bf16", layer="dispatch"),
    3: Shape("cfg3_full_layer_4k", tokens=8192, d_model=6144, latent=3072,
             n_experts=384, top_k=8, n_ranks=64, waves=3, expert_hidden=1536,
             shared_experts=2, shared_hidden=1536, act="bf16"),
    4: Shape("cfg4_zipf_skew", tokens=8192, d_model=6144, latent=3072,
             n_experts=384, top_k=8, n_ranks=64, waves=3, expert_hidden=1536,
             shared_experts=2, shared_hidden=1536, act="bf16", bias="zipf",
             receiver="hot_expert", layer="dispatch"),
    5: Shape("cfg5_long_context_64k", tokens=65536, d_model=6144, latent=3072,
             n_experts=384, top_k=8, n_ranks=64, waves=3, expert_hidden=1536,
             shared_experts=2, shared_hidden=1536, act="bf16", bias="segments",
             foreign="drawn"),
    # the expert width the pages' parameter counts imply (routed and shared
    # hidden 3072; about a third of the expert compute in the shared experts)
    6: Shape("cfg6_full_layer_4k_h3072", tokens=8192, d_model=6144, latent=3072,
             n_experts=384, top_k=8, n_ranks=64, waves=3, expert_hidden=3072,
             shared_experts=2, shared_hidden=3072, act="bf16"),
}

# Small bf16 workloads for element-by-element parity: several GEMM tiles in
# every dimension, ragged tails, every rank emulated.
MINI = {
    "mini_bf16": Shape("mini_bf16", tokens=333, d_model=512, latent=256,
                       n_experts=48, top_k=4, n_ranks=8, waves=3,
                       expert_hidden=128, shared_experts=2, shared_hidden=128,
                       act="bf16", emulate_all_ranks=True),
    # strong skew: both capacities bind
    "mini_bf16_skew": Shape("mini_bf16_skew", tokens=301, d_model=384,
                            latent=192, n_experts=24, top_k=3, n_ranks=4,
                            waves=3, expert_hidden=64, shared_experts=1,
                            shared_hidden=192, act="bf16",
                            emulate_all_ranks=True, bias="zipf", zipf_std=1.5),
    # segment-correlated routing, one wave of three experts
    "mini_bf16_seg": Shape("mini_bf16_seg", tokens=1100, d_model=256,
                           latent=128, n_experts=36, top_k=4, n_ranks=6,
                           waves=2, expert_hidden=64, shared_experts=2,
                           shared_hidden=64, act="bf16",
                           emulate_all_ranks=True, bias="segments",
                           segment_tokens=100, segment_hot=4),
    # long K (2048 and more) over few output tiles: every bf16 GEMM but the
    # shared experts' gate/up takes the tail split along K
    "mini_bf16_longk": Shape("mini_bf16_longk", tokens=300, d_model=2048,
                             latent=2048, n_experts=24, top_k=2, n_ranks=4,
                             waves=3, expert_hidden=1792, shared_experts=1,
                             shared_hidden=512, act="bf16",
                             emulate_all_ranks=True),
    # fp32 with ragged sizes everywhere
    "mini_f32": Shape("mini_f32", tokens=77, d_model=40, latent=24,
                      n_experts=12, top_k=3, n_ranks=3, waves=2,
                      expert_hidden=20, shared_experts=2, shared_hidden=12,
                      act="f32", emulate_all_ranks=True),
}


def get(cfg):
    """Shape for a config number (1..5) or a MINI name."""
    if isinstance(cfg, int):
        return CONFIGS[cfg]
    if isinstance(cfg, str) and cfg.isdigit():
        return CONFIGS[int(cfg)]
    return MINI[cfg]


def exact_fit(shape, pool_rows, expert_rows):
    """The shape with capacity factors that make the send cap exactly
    ``pool_rows`` and the receive cap exactly ``expert_rows`` (the largest
    demand of any pool and the largest arrivals at any expert, known once the
    counts are exchanged): nothing is dropped, and every fixed buffer is as
    small as that allows.  The factors stay exact rationals:
    ceil(f * T*k/R) = pool_rows for f = pool_rows*R / (T*k), and likewise for
    the receive cap over the balanced expert load R*T*k/E."""
    n = shape.tokens * shape.top_k
    return replace(shape, send_num=max(int(pool_rows), 1) * shape.n_ranks, send_den=max(n, 1),
                   recv_num=max(int(expert_rows), 1) * shape.n_experts, recv_den=max(shape.n_ranks * n, 1))


def with_tokens(shape, tokens):
    return replace(shape, tokens=tokens, name=f"{shape.name}_T{tokens}")
