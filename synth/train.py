"""Seeded synthetic inputs for one training step of the MoE layer.

Shapes and distributions only (no arithmetic of the layer).  Recipe: x,
the RMSNorm weight, the router weight and the correction bias exactly as
the inference workload of the same shape draws them (synth.gen); expert
weights ~ N(0, weight_std) rounded to bf16, in the canonical layout
[expert][gate [I, d], up [I, d], down [d, I]] (each expert drawn from its
own generator, so any expert can be regenerated alone); the output gradient
dout ~ N(0, 1) rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from .configs import MoEShape
from .gen import _randn, bias_vector, generate_router_inputs

ROLE_TRAIN_W, ROLE_DOUT = 41, 42


@dataclass
class TrainInputs:
    shape: MoEShape
    x: torch.Tensor          # [T, d] bf16
    norm_w: torch.Tensor     # [d] bf16
    w_router: torch.Tensor   # [E, d] bf16
    bias: torch.Tensor       # [E] fp32
    w: torch.Tensor          # [G * 3 * I * d] bf16, canonical layout
    dout: torch.Tensor       # [T, d] bf16

    def expert(self, e: int):
        """(gate [I, d], up [I, d], down [d, I]) views of expert e."""
        sh = self.shape
        I, d = sh.d_ff, sh.d_model
        base = self.w[e * 3 * I * d:(e + 1) * 3 * I * d]
        return base[:I * d].view(I, d), base[I * d:2 * I * d].view(I, d), base[2 * I * d:].view(d, I)


def expert_weights(shape: MoEShape, e: int, seed: int, device) -> torch.Tensor:
    I, d = shape.d_ff, shape.d_model
    return _randn((3 * I * d,), shape.weight_std, device, seed, ROLE_TRAIN_W, e).to(torch.bfloat16)


def generate_train(shape: MoEShape, seed: int = 0, device="cpu") -> TrainInputs:
    assert shape.fmt == "fp8" and not shape.dense
    x, norm_w, w_router = generate_router_inputs(shape, seed, device)
    bias = bias_vector(shape, seed, device)
    G = shape.n_experts + shape.n_shared
    per = 3 * shape.d_ff * shape.d_model
    w = torch.empty(G * per, dtype=torch.bfloat16, device=device)
    for e in range(G):
        w[e * per:(e + 1) * per] = expert_weights(shape, e, seed, device)
    dout = _randn(tuple(x.shape), 1.0, device, seed, ROLE_DOUT).to(torch.bfloat16)
    return TrainInputs(shape, x, norm_w, w_router, bias, w, dout)
