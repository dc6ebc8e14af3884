"""CPU oracle of the routing bias update (aux-loss-free load balancing).

Test infrastructure only: imported by tests/, the smoke check and the CPU
baseline of bench.py, never by the product path.

The router adds a per-expert correction bias to the sigmoid scores for the
top-k choice only ("Kimi-K2-Base", Mixture of experts, Load balancing: an
aux-loss-free selection bias, config topk_method noaux_tc).  The pages state
that the rule which adjusts that bias during training is not described.
Reading taken (the published aux-loss-free balancing rule, Wang et al. 2024,
"Auxiliary-Loss-Free Load Balancing Strategy for Mixture-of-Experts"):

* the load c_e of routed expert e over a training step is the number of
  top-k choices, over all tokens of the step, that picked e;
* after the step, every bias moves by a fixed speed u towards balance:
      b_e <- b_e + u * sign(cbar - c_e),   cbar = (sum_e c_e) / E,
  an under-loaded expert's bias rises, an over-loaded one's falls, and an
  expert exactly at the mean keeps its bias;
* the bias is fp32 (the dtype the router reads) and the update is one fp32
  addition of +u, -u or 0 to it.

The sign is decided on integers: sign(cbar - c_e) = sign(sum_e c_e - E c_e),
so no rounding enters the choice of direction.
"""
from __future__ import annotations

import numpy as np


def expert_load(ids: np.ndarray, n_experts: int) -> np.ndarray:
    """Loads c_e: how many entries of the top-k choice array ids [T, k]
    equal e, for 0 <= e < n_experts; entries outside that range (not a
    routed expert of this layer) are not counted.  int64 [n_experts]."""
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    keep = flat[(flat >= 0) & (flat < n_experts)]
    return np.bincount(keep, minlength=n_experts).astype(np.int64)


def load_direction(counts: np.ndarray) -> np.ndarray:
    """sign(cbar - c_e) in {-1, 0, +1} for every expert, from integer loads."""
    c = np.asarray(counts, dtype=np.int64)
    return np.sign(c.sum() - c.size * c).astype(np.int64)


def bias_update(bias: np.ndarray, counts: np.ndarray, speed: float) -> np.ndarray:
    """The bias after one step: fp32 bias + fp32(speed) * direction, one fp32
    rounding per expert (speed * direction is exact)."""
    b = np.asarray(bias, dtype=np.float32)
    step = np.float32(speed) * load_direction(counts).astype(np.float32)
    return (b + step).astype(np.float32)
