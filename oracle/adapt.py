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


def run_mla_oracle(inputs, tokens=None) -> dict:
    """MLA oracle forward on generated inputs (any device), on a host copy of
    the cache (the oracle writes the new positions into it; returned as
    "cache")."""
    import numpy as np
    from .mla_ref import MLAParams, mla_layer
    sh = inputs.shape
    p = MLAParams(d_model=sh.d_model, n_heads=sh.n_heads, q_lora=sh.q_lora, kv_lora=sh.kv_lora,
                  qk_nope=sh.qk_nope, qk_rope=sh.qk_rope, v_head=sh.v_head,
                  rope_theta=sh.rope_theta, rope_factor=sh.rope_factor,
                  rope_orig_len=sh.rope_orig_len, beta_fast=sh.beta_fast,
                  beta_slow=sh.beta_slow, mscale_all_dim=sh.mscale_all_dim, rms_eps=sh.rms_eps)
    w = {k: v.detach().cpu().numpy() for k, v in inputs.w.items()}
    w["g_in"] = to_f32(inputs.norm_w)
    w["g_qa"] = to_f32(inputs.g_qa)
    w["g_kva"] = to_f32(inputs.g_kva)
    cache = dict(codes=inputs.cache_codes.cpu().numpy().copy(),
                 scales=inputs.cache_scales.cpu().numpy().copy(),
                 rope=to_f32(inputs.cache_rope).copy())
    T = sh.tokens
    seq_of = np.arange(T) // sh.n_new
    pos_of = np.asarray(sh.cached, dtype=np.int64)[seq_of] + np.arange(T) % sh.n_new
    res = mla_layer(p, to_f32(inputs.x), w, seq_of, pos_of, cache, tokens=tokens)
    res.update(cache=cache, seq_of=seq_of, pos_of=pos_of, params=p)
    return res


class LazyExperts:
    """Expert weights of a training workload fetched from the device one
    expert at a time (float32 arrays of the bf16 values)."""

    def __init__(self, inputs, which):
        self.inputs, self.which = inputs, which
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            g, u, d = self.inputs.expert(e)
            self.cache[e] = to_f32({"gate": g, "up": u, "down": d}[self.which])
        return self.cache[e]


def train_oracle_inputs(inputs):
    """(params, x, norm_w, bias, TrainWeights, dout) of a training workload,
    the expert weights fetched lazily."""
    from .train_ref import TrainWeights
    p = params_from_shape(inputs.shape)
    W = TrainWeights(gate=LazyExperts(inputs, "gate"), up=LazyExperts(inputs, "up"),
                     down=LazyExperts(inputs, "down"), w_router=to_f32(inputs.w_router))
    return (p, to_f32(inputs.x), to_f32(inputs.norm_w), inputs.bias.detach().cpu().numpy(), W,
            to_f32(inputs.dout))
