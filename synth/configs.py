"""Workload shapes for the Kimi K2 sparse-MoE feed-forward layer.

Each shape names the layer's dimensions and the synthetic input recipe.  The
K2 numbers come from the released configuration printed on the
"Kimi K2 · Architecture" page (config.json: hidden_size 7168,
n_routed_experts 384, n_shared_experts 1, num_experts_per_tok 8,
moe_intermediate_size 2048, intermediate_size 18432, n_group 1, topk_group 1,
routed_scaling_factor 2.827, norm_topk_prob true, rms_norm_eps 1e-6,
quantization_config fp8 / e4m3 / weight_block_size [128, 128] /
activation_scheme dynamic).

This module holds shapes and distribution parameters only: no arithmetic of
the layer itself.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

FMT_F32 = "f32"   # fp32 activations and weights, no quantisation
FMT_FP8 = "fp8"   # bf16 activations, FP8 e4m3 weights with 128x128 fp32 block scales

# config.json: routed_scaling_factor
K2_ROUTED_SCALING = 2.827
# config.json: rms_norm_eps
K2_RMS_EPS = 1e-6


@dataclass(frozen=True)
class MoEShape:
    name: str
    tokens: int
    d_model: int
    n_experts: int          # routed experts
    n_shared: int           # always-on experts (weight 1)
    top_k: int
    d_ff: int               # hidden features of one expert
    fmt: str
    routed_scaling: float = K2_ROUTED_SCALING
    rms_eps: float = K2_RMS_EPS
    norm_topk_prob: bool = True
    dense: bool = False     # one expert, no router, weight 1 (the first block's MLP)
    # input recipe
    x_std: float = 1.0
    gamma_std: float = 0.0        # RMSNorm weight: 1 (0.0) or ~N(1, gamma_std)
    weight_std: float = 0.02
    bias_std: float = 0.01
    bias_recipe: str = "normal"   # "normal": N(0, bias_std); "zipf": -beta*ln(rank)
    zipf_beta: float = 0.0

    @property
    def n_pairs(self) -> int:
        return self.tokens * self.top_k

    def with_tokens(self, tokens: int) -> "MoEShape":
        return replace(self, tokens=tokens)


# 64 tokens, d 256, 16 routed + 1 shared, top-4, hidden 128, fp32 throughout.
TINY = MoEShape("tiny", tokens=64, d_model=256, n_experts=16, n_shared=1, top_k=4,
                d_ff=128, fmt=FMT_F32)

# One K2 MoE layer, 64-token decode step (batch 64 x 1 position).
K2_DECODE = MoEShape("k2_decode", tokens=64, d_model=7168, n_experts=384, n_shared=1,
                     top_k=8, d_ff=2048, fmt=FMT_FP8)

# 8192-token prefill (batch 2 x 4096 positions), same layer.
K2_PREFILL = K2_DECODE.with_tokens(8192)
K2_PREFILL = replace(K2_PREFILL, name="k2_prefill")

# 16384 tokens with a correction bias that gives Zipf-like (s = 1.1) expert
# popularity.  beta is fitted by oracle/fit_zipf_beta.py and frozen here.
K2_SKEWED = replace(K2_DECODE, name="k2_skewed", tokens=16384, bias_recipe="zipf",
                    zipf_beta=0.0434)

# The first block's dense SwiGLU (7168 -> 18432 -> 7168) run as one expert.
K2_DENSE = MoEShape("k2_dense", tokens=4096, d_model=7168, n_experts=1, n_shared=0,
                    top_k=1, d_ff=18432, fmt=FMT_FP8, routed_scaling=1.0, dense=True)

# One GPU's share of the layer under 8-way expert parallelism: 48 of the 384
# routed experts per GPU, and 8192 tokens on each of 8 GPUs send on average
# 8 * 8192 * 8 / 384 = 1365 rows to each local expert.  Modelled as a
# 48-expert layer with 8192 tokens and top-8, so the grouped GEMMs see the
# same rows per expert (the shared expert runs over the GPU's own 8192 tokens).
K2_EP8_SHARD = replace(K2_DECODE, name="k2_ep8_shard", tokens=8192, n_experts=48)

ALL = {s.name: s for s in (TINY, K2_DECODE, K2_PREFILL, K2_SKEWED, K2_DENSE, K2_EP8_SHARD)}


def small_fp8(tokens=48, d_model=256, n_experts=8, n_shared=1, top_k=2, d_ff=256,
              **kw) -> MoEShape:
    """A K2-format (bf16 + FP8) layer small enough for the CPU oracle in seconds."""
    return MoEShape("small_fp8", tokens=tokens, d_model=d_model, n_experts=n_experts,
                    n_shared=n_shared, top_k=top_k, d_ff=d_ff, fmt=FMT_FP8, **kw)
