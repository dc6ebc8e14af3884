"""Marshal generated torch inputs into the oracle's numpy arguments.

TEST INFRASTRUCTURE ONLY.  Copies tensors to host memory and converts bf16
to the float32 values they hold (exact); no arithmetic of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from .moe_ref import LayerParams, moe_layer, params_from_shape


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()


class ExpertFetcher:
    """expert(e) -> numpy weights, copying one expert at a time from ``inputs``."""

    def __init__(self, inputs):
        self.inp = inputs

    def __call__(self, e: int) -> dict:
        out = {}
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            t = getattr(self.inp, name)
            out[name] = None if t is None else t[e].detach().to("cpu").numpy()
        return out


def run_oracle(inputs, tokens=None) -> dict:
    """Oracle forward on generated inputs (any device)."""
    p: LayerParams = params_from_shape(inputs.shape)
    x = to_f32(inputs.x)
    norm_w = to_f32(inputs.norm_w)
    wr = None if inputs.w_router is None else to_f32(inputs.w_router)
    bias = None if inputs.bias is None else to_f32(inputs.bias)
    return moe_layer(p, x, norm_w, wr, bias, ExpertFetcher(inputs), tokens=tokens)
