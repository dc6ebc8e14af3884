"""Seeded synthetic inputs: determinism, per-expert independence and recipe.

CPU only; small shapes.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle.fit_zipf_beta import load_slope
from oracle.fp8 import e4m3_decode

SHAPE = synth.small_fp8(tokens=8, d_model=256, n_experts=16, n_shared=1, top_k=2, d_ff=128)
FIELDS = ("x", "norm_w", "w_router", "bias", "w_gate", "w_up", "w_down", "s_gate", "s_up",
          "s_down")


def _bytes(t):
    return t.contiguous().view(torch.uint8) if t.dtype != torch.uint8 else t


def test_same_seed_gives_identical_inputs():
    a = synth.generate(SHAPE, seed=5)
    b = synth.generate(SHAPE, seed=5)
    for f in FIELDS:
        assert torch.equal(_bytes(getattr(a, f)), _bytes(getattr(b, f))), f


def test_different_seed_changes_every_random_tensor():
    a = synth.generate(SHAPE, seed=5)
    b = synth.generate(SHAPE, seed=6)
    for f in ("x", "w_router", "bias", "w_gate", "w_up", "w_down"):
        assert not torch.equal(_bytes(getattr(a, f)), _bytes(getattr(b, f))), f


def test_expert_weights_do_not_depend_on_the_expert_count():
    small = dataclasses.replace(SHAPE, n_shared=0)
    big = dataclasses.replace(SHAPE, n_experts=32, n_shared=0)
    a = synth.generate(small, seed=3)
    b = synth.generate(big, seed=3)
    for f in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        assert torch.equal(getattr(a, f), getattr(b, f)[:16]), f


def test_router_inputs_match_the_full_generator():
    full = synth.generate(SHAPE, seed=9, tokens=12)
    x, norm_w, w_router = synth.generate_router_inputs(SHAPE, seed=9, tokens=12)
    assert torch.equal(_bytes(x), _bytes(full.x))
    assert torch.equal(_bytes(norm_w), _bytes(full.norm_w))
    assert torch.equal(_bytes(w_router), _bytes(full.w_router))


def test_with_workload_keeps_the_weights():
    base = synth.generate(SHAPE, seed=2)
    other = synth.with_workload(base, SHAPE, seed=4, tokens=20)
    assert other.x.shape == (20, SHAPE.d_model)
    assert other.w_gate is base.w_gate and other.w_router is base.w_router
    assert not torch.equal(_bytes(other.bias), _bytes(base.bias))


def test_block_quantisation_recipe():
    g = torch.Generator().manual_seed(0)
    w = torch.randn(256, 384, generator=g) * 0.02
    codes, scales = synth.block_quantize_weight(w)
    dec = torch.from_numpy(e4m3_decode(codes.numpy()))
    blocks = w.view(2, 128, 3, 128).abs().amax(dim=(1, 3))
    assert torch.equal(scales, blocks / 448.0)
    # the largest element of every block maps to code magnitude 448
    dmax = dec.view(2, 128, 3, 128).abs().amax(dim=(1, 3))
    assert torch.all(dmax == 448.0)
    # dequantised weights within half an e4m3 step (relative 2^-4) of the originals
    back = dec * scales.repeat_interleave(128, 0).repeat_interleave(128, 1)
    big = w.abs() > scales.repeat_interleave(128, 0).repeat_interleave(128, 1) * 2.0 ** -6
    rel = ((back - w).abs() / w.abs())[big]
    assert rel.max() <= 2.0 ** -4 + 1e-6


def test_skewed_bias_is_minus_beta_log_rank():
    shape = synth.K2_SKEWED
    b = synth.bias_vector(shape, 0, "cpu").double().numpy()
    r = np.sort(np.exp(-b / shape.zipf_beta))
    assert np.allclose(r, np.arange(1, shape.n_experts + 1), rtol=1e-5)
    assert np.array_equal(synth.bias_vector(shape, 0, "cpu").numpy(),
                          synth.bias_vector(shape, 0, "cpu").numpy())


def test_normal_bias_scale():
    shape = dataclasses.replace(SHAPE, n_experts=4096)
    b = synth.bias_vector(shape, 1, "cpu").numpy()
    assert abs(b.std() / shape.bias_std - 1.0) < 0.05


@pytest.mark.parametrize("s", [0.8, 1.1, 1.5])
def test_load_slope_recovers_a_zipf_exponent(s):
    r = np.arange(1, 385)
    loads = np.round(1e6 * r ** -s)
    assert abs(load_slope(loads) + s) < 1e-3


def test_gamma_recipe():
    """gamma is 1 by default and ~N(1, gamma_std) in the layer dtype when asked
    for; with_workload draws it from the new shape and keeps the base's
    otherwise."""
    a = synth.generate(SHAPE, seed=3)
    assert torch.equal(a.norm_w, torch.ones_like(a.norm_w)) and a.norm_w.dtype == torch.bfloat16
    shp = dataclasses.replace(synth.small_fp8(tokens=8, d_model=4096), gamma_std=0.1)
    g = synth.generate(shp, seed=3).norm_w.float()
    assert abs(float(g.mean()) - 1.0) < 0.01 and abs(float(g.std()) - 0.1) < 0.01
    tiny = synth.generate(dataclasses.replace(synth.TINY, gamma_std=0.1), seed=3).norm_w
    assert tiny.dtype == torch.float32 and float(tiny.std()) > 0.05
    w = synth.with_workload(a, dataclasses.replace(SHAPE, gamma_std=0.1), seed=4)
    assert not torch.equal(w.norm_w, a.norm_w)
    assert synth.with_workload(a, SHAPE, seed=4).norm_w is a.norm_w
