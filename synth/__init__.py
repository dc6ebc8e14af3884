"""Seeded synthetic workloads for the K2 MoE layer and the MLA attention sub-layer
(shapes and input recipe only)."""
from .configs import (ALL, FMT_F32, FMT_FP8, K2_DECODE, K2_DENSE, K2_EP8_SHARD, K2_PREFILL,
                      K2_SKEWED, TINY, MoEShape, small_fp8)
from .mla import (MLA_K2_DECODE, MLA_K2_PREFILL, MLAInputs, MLAShape, generate_mla,
                  small_mla)
from .balance import bias_values, expert_loads, topk_choices
from .train import TrainInputs, generate_train
from .gen import (MoEInputs, bias_vector, block_quantize_weight, generate,
                  generate_router_inputs, with_workload)

__all__ = ["ALL", "FMT_F32", "FMT_FP8", "K2_DECODE", "K2_DENSE", "K2_EP8_SHARD", "K2_PREFILL",
           "K2_SKEWED",
           "TINY", "MoEShape", "small_fp8", "MoEInputs", "block_quantize_weight", "generate",
           "generate_router_inputs", "bias_vector",
           "with_workload", "MLAShape", "MLAInputs", "MLA_K2_DECODE", "MLA_K2_PREFILL",
           "generate_mla", "small_mla", "topk_choices", "expert_loads", "bias_values",
           "TrainInputs", "generate_train"]
