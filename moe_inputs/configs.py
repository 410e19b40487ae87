"""Layer configurations (shapes and routing rules) for the synthetic workloads.

Field names follow the C struct ``moe_config`` in ``include/moe.h``.  The
five full-size workloads are the ones the layer is measured on; the SMALL
variants keep each workload's structure (routing rule, groups, shared
experts, heads, Zipf hot experts) at sizes the CPU oracle finishes in
seconds, while still spanning several GEMM tiles and a ragged tail.
"""
from dataclasses import dataclass, replace, asdict

DROP_NONE, DROP_CAPACITY, DROP_AFFINITY = 0, 1, 2
ROUTE_TOKEN_CHOICE, ROUTE_EXPERT_CHOICE = 0, 1
ACT_RELU, ACT_SWIGLU = 0, 1
F32, BF16 = 0, 1


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                  # tokens
    d_model: int
    n_heads: int            # H routing heads (1 = ordinary MoE)
    d_head: int             # expert input width d_e (= d_model when H == 1)
    n_experts: int          # routed experts in total, H * E_h
    top_k: int              # experts chosen per head
    n_groups: int = 0       # group-limited routing: groups per head (0 = off)
    topk_groups: int = 0    # groups kept per token
    renorm: int = 0         # 1: chosen gates divided by their sum
    drop: int = DROP_NONE
    capacity: int = 0       # integer C for DROP_CAPACITY
    keep_num: int = 1       # DROP_AFFINITY keeps ceil(keep_num * n_e / keep_den)
    keep_den: int = 1
    d_ff: int = 0
    act: int = ACT_SWIGLU
    n_shared: int = 0
    latent_proj: int = 0    # 1: z = x W_in^T before routing, y = o W_out^T + x after
    residual: int = 1       # 1: combine adds the layer input
    act_dtype: int = BF16
    router_dtype: int = BF16
    route_mode: int = ROUTE_TOKEN_CHOICE  # expert choice: each expert keeps its top-`capacity` tokens
    sel_bias_gate: int = 0  # with a selection bias: 1 the gate is p + b, 0 the gate is p
    seq_len: int = 0        # > 0: per-sequence balance statistic over sequences of seq_len tokens
    # input recipe (not part of the C struct)
    zipf_s: float = 0.0     # > 0: router bias b_e = -s ln(e+1) per head
    sel_bias_steps: int = 0  # > 0: selection bias b_e = 0.001 * n_e, n_e uniform in [-steps, steps]
    seed: int = 0
    tag: int = 0            # config tag mixed into every tensor's stream

    @property
    def e_per_head(self):
        return self.n_experts // self.n_heads

    @property
    def k_total(self):
        """Assignment slots per token: H * top_k, or one per expert with expert choice."""
        return self.n_experts if self.route_mode == ROUTE_EXPERT_CHOICE else self.n_heads * self.top_k

    @property
    def d_latent(self):
        return self.n_heads * self.d_head

    @property
    def d_router(self):
        return self.d_head

    def c_fields(self):
        d = asdict(self)
        for k in ("name", "zipf_s", "sel_bias_steps", "seed", "tag"):
            d.pop(k)
        return d

    def with_(self, **kw):
        return replace(self, **kw)


# Tiny GShard-style MoE, fp32: top-2, capacity factor 1.25 -> C = ceil(1.25*256*2/8) = 80.
C0 = MoEConfig("c0_gshard_tiny_f32", T=256, d_model=128, n_heads=1, d_head=128,
               n_experts=8, top_k=2, drop=DROP_CAPACITY, capacity=80, d_ff=256,
               act=ACT_RELU, act_dtype=F32, router_dtype=F32, tag=0)
# Coarse MoE, bf16 with an fp32 router: top-2 renormalised, no drop, SwiGLU 14336.
C1 = MoEConfig("c1_coarse_t4096_d4096_e8", T=4096, d_model=4096, n_heads=1, d_head=4096,
               n_experts=8, top_k=2, renorm=1, drop=DROP_NONE, d_ff=14336,
               act=ACT_SWIGLU, act_dtype=BF16, router_dtype=F32, tag=1)
# Fine-grained MoE + 2 shared experts, capacity factor 1.0 -> C = ceil(8192*6/64) = 768.
C2 = MoEConfig("c2_fine_shared_t8192_d2048_e64", T=8192, d_model=2048, n_heads=1, d_head=2048,
               n_experts=64, top_k=6, drop=DROP_CAPACITY, capacity=768, d_ff=1408,
               n_shared=2, zipf_s=1.1, tag=2)
# Group-limited: 160 experts in 8 groups of 20, top-3 groups then top-6, keep 90 % per expert.
C3 = MoEConfig("c3_group_limited_t8192_d5120_e160", T=8192, d_model=5120, n_heads=1,
               d_head=5120, n_experts=160, top_k=6, n_groups=8, topk_groups=3,
               drop=DROP_AFFINITY, keep_num=9, keep_den=10, d_ff=1536, n_shared=2, tag=3)
# Multi-head latent MoE: 8 heads x 256 latent, 16 experts per head, top-1 per head.
C4 = MoEConfig("c4_multihead_latent_t16384_d2048_h8", T=16384, d_model=2048, n_heads=8,
               d_head=256, n_experts=128, top_k=1, drop=DROP_NONE, d_ff=512,
               latent_proj=1, zipf_s=1.0, tag=4)

CONFIGS = [C0, C1, C2, C3, C4]

# Oracle-sized variants with the same structure.
SMALL = [
    C0,
    C1.with_(name="c1s", T=300, d_model=256, d_head=256, d_ff=384, tag=11),
    C2.with_(name="c2s", T=520, d_model=256, d_head=256, n_experts=16, d_ff=192,
             capacity=(520 * 6 + 15) // 16, tag=12),
    C3.with_(name="c3s", T=400, d_model=320, d_head=320, n_experts=40, n_groups=8,
             topk_groups=3, d_ff=192, tag=13),
    C4.with_(name="c4s", T=333, d_model=256, n_heads=4, d_head=64, n_experts=64,
             d_ff=128, tag=14),
]


# Routing variants on the fine-grained workload's shapes.
# Expert choice: every expert keeps its top-768 tokens (= T*6/64: as many rows as
# top-6 token choice at capacity factor 1.0).
C2EC = C2.with_(name="c2ec_expert_choice_t8192_d2048_e64", route_mode=ROUTE_EXPERT_CHOICE, capacity=768, tag=5)
# Balancing bias (selection only) with no dropping, and the per-sequence balance
# statistic over two 4096-token sequences.
C2V3 = C2.with_(name="c2v3_balancing_bias_t8192_d2048_e64", drop=DROP_NONE, capacity=0, sel_bias_steps=8,
                seq_len=4096, tag=6)
VARIANTS = [C2EC, C2V3]

SMALL_VARIANTS = [
    C2EC.with_(name="c2ec_s", T=520, d_model=256, d_head=256, n_experts=16, d_ff=192,
               capacity=(520 * 6 + 15) // 16, tag=15),
    C2V3.with_(name="c2v3_s", T=520, d_model=256, d_head=256, n_experts=16, d_ff=192, seq_len=260, tag=16),
    # group-limited selection on the biased keys, bias inside renormalised-free gates, fp32
    C3.with_(name="c3v3_s", T=400, d_model=320, d_head=320, n_experts=40, n_groups=8, topk_groups=3, d_ff=192,
             drop=DROP_NONE, sel_bias_steps=8, sel_bias_gate=1, seq_len=100, n_shared=0, tag=17),
    # expert choice in float32 with a ragged T and C > T / E
    C0.with_(name="c0ec_f32", T=199, route_mode=ROUTE_EXPERT_CHOICE, capacity=70, tag=18),
]


def config_by_name(name):
    for c in CONFIGS + SMALL + VARIANTS + SMALL_VARIANTS:
        if c.name == name:
            return c
    raise KeyError(name)
