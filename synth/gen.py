"""Seeded synthetic inputs for the K2 MoE layer.

Every tensor role gets its own torch generator, seeded from
``numpy.random.SeedSequence([master, role, i, j])``, so any expert can be
regenerated alone.  Values are drawn on the requested device; CPU and GPU
draws of the same seed differ, so a comparison always copies one set of
generated tensors to wherever it is needed.

Input recipe (the distributions of the workloads being modelled):

* x ~ N(0, 1), stored bf16 (fp32 for the fp32 format);
* RMSNorm weight gamma = 1 (the norm's initial value; every benchmark
  workload), or gamma ~ N(1, gamma_std) for parity cases that exercise it;
* router weight ~ N(0, 0.02), bf16 [E, d];
* correction bias ~ N(0, 0.01) fp32, or -beta * ln(rank) with rank a seeded
  permutation of 1..E for the skewed workload;
* expert weights ~ N(0, 0.02) in nn.Linear [out, in] layout.  For the FP8
  format each 128x128 block is stored as e4m3 codes with one fp32 scale,
  scale = block amax / 448, codes = e4m3(clamp(w / scale, +-448)).  This is
  how the checkpoint was made, not a step of the layer: the conversion uses
  torch's own float8_e4m3fn cast, and the layer only ever sees the codes and
  scales.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import FMT_F32, FMT_FP8, MoEShape

ROLE_X, ROLE_ROUTER, ROLE_BIAS, ROLE_EXPERT, ROLE_RANK, ROLE_NORM = 1, 2, 3, 4, 5, 6
MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2
FP8_MAX = 448.0
BLOCK = 128


def _seed(master: int, *key: int) -> int:
    ss = np.random.SeedSequence([int(master), *[int(k) for k in key]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def _gen(device, master: int, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(master, *key))
    return g


def _randn(shape, std: float, device, master: int, *key: int) -> torch.Tensor:
    g = _gen(device, master, *key)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def block_quantize_weight(w: torch.Tensor):
    """fp32 [N, K] -> (uint8 e4m3 codes [N, K], fp32 scales [N/128, K/128])."""
    n, k = w.shape
    assert n % BLOCK == 0 and k % BLOCK == 0
    blk = w.view(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = amax / FP8_MAX
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    v = (blk / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, k)
    return codes.contiguous(), scale.contiguous()


@dataclass
class MoEInputs:
    shape: MoEShape
    x: torch.Tensor                    # [T, d] bf16 (fp32 for FMT_F32)
    norm_w: torch.Tensor               # [d]   same dtype as x
    w_router: Optional[torch.Tensor]   # [E, d] bf16 / fp32; None when dense
    bias: Optional[torch.Tensor]       # [E] fp32; None when dense
    # expert weights, experts stacked along dim 0 (routed 0..E-1, then shared)
    w_gate: torch.Tensor               # [NE, I, d]  uint8 codes or fp32
    w_up: torch.Tensor                 # [NE, I, d]
    w_down: torch.Tensor               # [NE, d, I]
    s_gate: Optional[torch.Tensor]     # [NE, I/128, d/128] fp32 (FP8 only)
    s_up: Optional[torch.Tensor]
    s_down: Optional[torch.Tensor]     # [NE, d/128, I/128]

    def to(self, device) -> "MoEInputs":
        mv = lambda t: None if t is None else t.to(device)
        return MoEInputs(self.shape, mv(self.x), mv(self.norm_w), mv(self.w_router),
                         mv(self.bias), mv(self.w_gate), mv(self.w_up), mv(self.w_down),
                         mv(self.s_gate), mv(self.s_up), mv(self.s_down))

    def expert_numpy(self, e: int) -> dict:
        """One expert's weights as numpy arrays (copied to host)."""
        out = {}
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            t = getattr(self, name)
            out[name] = None if t is None else t[e].detach().cpu().numpy()
        return out


def norm_weight(shape: MoEShape, seed: int, device, dtype) -> torch.Tensor:
    """RMSNorm weight gamma [d]: ones, or ~N(1, gamma_std) rounded to ``dtype``."""
    if shape.gamma_std == 0.0:
        return torch.ones(shape.d_model, dtype=dtype, device=device)
    g = _randn((shape.d_model,), shape.gamma_std, device, seed, ROLE_NORM) + 1.0
    return g.to(dtype)


def bias_vector(shape: MoEShape, seed: int, device) -> torch.Tensor:
    E = shape.n_experts
    if shape.bias_recipe == "normal":
        return _randn((E,), shape.bias_std, device, seed, ROLE_BIAS)
    if shape.bias_recipe == "zipf":
        g = _gen("cpu", seed, ROLE_RANK)
        rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
        return (-shape.zipf_beta * torch.log(rank)).to(torch.float32).to(device)
    raise ValueError(shape.bias_recipe)


def generate_router_inputs(shape: MoEShape, seed: int = 0, device="cpu",
                           tokens: Optional[int] = None):
    """(x, norm_w, w_router) exactly as generate() draws them, without experts."""
    T = shape.tokens if tokens is None else tokens
    act_dtype = torch.bfloat16 if shape.fmt == FMT_FP8 else torch.float32
    x = _randn((T, shape.d_model), shape.x_std, device, seed, ROLE_X).to(act_dtype)
    norm_w = norm_weight(shape, seed, device, act_dtype)
    w_router = _randn((shape.n_experts, shape.d_model), shape.weight_std, device, seed,
                      ROLE_ROUTER).to(act_dtype)
    return x, norm_w, w_router


def generate(shape: MoEShape, seed: int = 0, device="cpu", tokens: Optional[int] = None) -> MoEInputs:
    """Seeded inputs for ``shape`` (optionally with a different token count)."""
    T = shape.tokens if tokens is None else tokens
    d, E, I = shape.d_model, shape.n_experts, shape.d_ff
    NE = E + shape.n_shared
    fp8 = shape.fmt == FMT_FP8
    act_dtype = torch.bfloat16 if fp8 else torch.float32

    x = _randn((T, d), shape.x_std, device, seed, ROLE_X).to(act_dtype)
    norm_w = norm_weight(shape, seed, device, act_dtype)
    if shape.dense:
        w_router = bias = None
    else:
        w_router = _randn((E, d), shape.weight_std, device, seed, ROLE_ROUTER).to(act_dtype)
        bias = bias_vector(shape, seed, device)

    wdt = torch.uint8 if fp8 else torch.float32
    w_gate = torch.empty((NE, I, d), dtype=wdt, device=device)
    w_up = torch.empty((NE, I, d), dtype=wdt, device=device)
    w_down = torch.empty((NE, d, I), dtype=wdt, device=device)
    if fp8:
        s_gate = torch.empty((NE, I // BLOCK, d // BLOCK), dtype=torch.float32, device=device)
        s_up = torch.empty_like(s_gate)
        s_down = torch.empty((NE, d // BLOCK, I // BLOCK), dtype=torch.float32, device=device)
    else:
        s_gate = s_up = s_down = None
    for e in range(NE):
        for mat, (wt, st, shp) in enumerate(((w_gate, s_gate, (I, d)), (w_up, s_up, (I, d)),
                                             (w_down, s_down, (d, I)))):
            w = _randn(shp, shape.weight_std, device, seed, ROLE_EXPERT, e, mat)
            if fp8:
                codes, scales = block_quantize_weight(w)
                wt[e].copy_(codes)
                st[e].copy_(scales)
            else:
                wt[e].copy_(w)
            del w
    return MoEInputs(shape, x, norm_w, w_router, bias, w_gate, w_up, w_down, s_gate, s_up, s_down)


def with_workload(base: MoEInputs, shape: MoEShape, seed: int = 0,
                  tokens: Optional[int] = None) -> MoEInputs:
    """Inputs of ``shape`` that reuse ``base``'s expert and router weights.

    Expert and router weights depend only on the seed and the layer
    dimensions, so workloads of one layer (decode, prefill, skewed routing)
    share them; x is drawn for the new token count, the bias from the new
    shape's recipe, and gamma from it when it asks for a non-unit one.
    """
    b = base.shape
    assert (b.d_model, b.n_experts, b.n_shared, b.d_ff, b.fmt) == \
        (shape.d_model, shape.n_experts, shape.n_shared, shape.d_ff, shape.fmt)
    device = base.x.device
    T = shape.tokens if tokens is None else tokens
    act_dtype = base.x.dtype
    x = _randn((T, shape.d_model), shape.x_std, device, seed, ROLE_X).to(act_dtype)
    bias = None if shape.dense else bias_vector(shape, seed, device)
    norm_w = base.norm_w if shape.gamma_std == 0.0 else norm_weight(shape, seed, device,
                                                                     act_dtype)
    return MoEInputs(shape, x, norm_w, base.w_router, bias, base.w_gate, base.w_up,
                     base.w_down, base.s_gate, base.s_up, base.s_down)
