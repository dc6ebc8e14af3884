"""Pins for the CPU oracle: page numbers, closed forms, invariants, brute force.

Every function in oracle/moe_ref.py is pinned here to something other than
itself: parameter counts printed on the pages, library routines for textbook
pieces (RMSNorm, sigmoid, SiLU), brute-force enumeration of the top-k sets and
of the permutation, closed-form special cases (a dense SwiGLU, hand-built
weights whose SwiGLU output is known), and invariants the method fixes
(weights sum to the routed scaling factor, the correction bias moves the
selection only, token and expert relabelling, power-of-two scale changes).
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import moe_ref as R
from oracle.adapt import run_oracle, to_f32
from oracle.fp8 import bf16_round, e4m3_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "param_counts.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, value = line.split()[:2]
        vals[name] = float(value) if "." in value else int(value)
    return vals


# ------------------------------------------------------------------ shapes ---
def test_layer_shape_reproduces_page_parameter_counts():
    g = _golden()
    s = synth.K2_DECODE
    d, E, S, I, k = s.d_model, s.n_experts, s.n_shared, s.d_ff, s.top_k
    Id = synth.K2_DENSE.d_ff
    vocab = 163840
    per_expert = 3 * I * d
    assert per_expert == 44_040_192
    dense_mlp = 3 * d * Id
    assert dense_mlp == g["dense_mlp"]
    # MLA from the released config (q latent 1536, kv latent 512, 64 heads,
    # qk 128 + 64 rotary, v 128): pins the dense block independently
    mla = (d * 1536 + 1536 + 1536 * 64 * 192 + d * (512 + 64) + 512 + 512 * 64 * (128 + 128)
           + 64 * 128 * d)
    assert mla == g["dense_attention"]
    assert mla + 2 * d + dense_mlp == g["dense_block"]
    moe_block = mla + 2 * d + (E + S) * per_expert + E * d + E
    assert moe_block == (g["transformer_blocks"] - g["dense_block"]) // 60
    assert (g["transformer_blocks"] - g["dense_block"]) % 60 == 0
    assert round(moe_block / 1e9, 2) == g["largest_layer_billions"]
    total = vocab * d + g["dense_block"] + 60 * moe_block + d + d * vocab
    assert total == g["model_total"]
    active_non_emb = g["dense_block"] + 60 * (mla + 2 * d + (k + S) * per_expert + E * d + E) + d
    assert round(active_non_emb / 1e9, 2) == g["active_non_embedding_billions"]
    assert round((active_non_emb + 2 * vocab * d) / 1e9, 1) == g["active_billions"]
    # one byte per FP8 matrix weight; embedding, head, norms, router in bf16
    bf16_params = 2 * vocab * d + 61 * 2 * d + d + 60 * E * d
    assert round((total + bf16_params) / 2 ** 30, 1) == g["whole_model_gib"]
    assert round(dense_mlp / 2 ** 20) == g["mlp_weight_mib"]


# ---------------------------------------------------------------- RMSNorm ---
def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 1, (32, 512)).astype(np.float32)
    gamma = rng.normal(1, 0.1, 512).astype(np.float32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (512,),
                                       torch.from_numpy(gamma).double(), eps=1e-6).numpy()
    h = R.rmsnorm(x, gamma, 1e-6, round_bf16=False)
    np.testing.assert_allclose(h, ref, rtol=4e-7, atol=0)
    hb = R.rmsnorm(x, gamma, 1e-6, round_bf16=True)
    assert np.array_equal(hb, bf16_round(h))


def test_rmsnorm_constant_row_closed_form():
    for c in (0.5, 3.0, -7.25, 1e-3):
        x = np.full((1, 256), c, np.float32)
        h = R.rmsnorm(x, np.ones(256, np.float32), 1e-6, round_bf16=False)
        expect = c / math.sqrt(c * c + 1e-6)
        np.testing.assert_allclose(h, expect, rtol=3e-7)


# --------------------------------------------------- activation quantiser ---
def test_quantize_scale_and_amax_code():
    rng = np.random.default_rng(1)
    a = rng.normal(0, 3, (16, 384)).astype(np.float32)
    codes, scales = R.quantize_1x128(a)
    blk = np.abs(a.reshape(16, 3, 128))
    amax = blk.max(axis=2)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    # the largest element of every block maps to +-448 (code 0x7E / 0xFE)
    c3 = codes.reshape(16, 3, 128)
    for r in range(16):
        for b in range(3):
            j = int(np.argmax(blk[r, b]))
            assert c3[r, b, j] & 0x7F == 0x7E


def test_quantize_error_bound_and_zero_block():
    rng = np.random.default_rng(2)
    a = rng.normal(0, 1, (8, 256)).astype(np.float32)
    a[3, 128:] = 0.0
    codes, scales = R.quantize_1x128(a)
    assert scales[3, 1] == 1.0 and np.all(codes[3, 128:] == 0)
    deq = R.dequantize_1x128(codes, scales)
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    err = np.abs(deq - a)
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 * scale below 2^-6
    bound = np.maximum(np.abs(a) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantize_power_of_two_rescale_keeps_codes():
    rng = np.random.default_rng(3)
    a = rng.normal(0, 1, (4, 256)).astype(np.float32)
    c1, s1 = R.quantize_1x128(a)
    c2, s2 = R.quantize_1x128(a * np.float32(8.0))
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * 8)


def test_quantize_exact_values():
    # amax 448 gives scale 1, so every e4m3-representable value maps to itself
    vals = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float32)
    row = np.zeros(128, np.float32)
    row[:127] = vals
    codes, scales = R.quantize_1x128(row[None])
    assert scales[0, 0] == 1.0
    assert np.array_equal(codes[0, :127], np.arange(0, 0x7F, dtype=np.uint8))


def test_weight_dequant_block_layout():
    codes = np.full((256, 384), 0x38, np.uint8)       # every code is 1.0
    scales = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    w = R.dequantize_weight(codes, scales)
    for i in range(2):
        for j in range(3):
            assert np.all(w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] == scales[i, j])


# ------------------------------------------------------------------ router ---
def test_router_logits_orientation():
    rng = np.random.default_rng(4)
    W = rng.normal(0, 0.02, (16, 64)).astype(np.float32)
    eye = np.eye(64, dtype=np.float32)
    z = R.router_logits(eye, W)          # token j = basis vector j -> column j of W
    assert z.shape == (64, 16)
    assert np.array_equal(z, W.T)


def test_sigmoid_matches_scipy():
    z = np.linspace(-30, 30, 1001).astype(np.float32)
    s = R.sigmoid_scores(z)
    assert s[500] == np.float32(0.5)
    np.testing.assert_allclose(s, scipy.special.expit(z.astype(np.float64)), rtol=1e-7)


def test_select_topk_small_example_and_ties():
    sb = np.array([[0.1, 0.5, 0.5, 0.3, 0.5]], np.float32)
    ids, gap = R.select_topk(sb, 2)
    assert ids.tolist() == [[1, 2]] and gap[0] == 0.0     # 3-way tie: lowest ids win
    ids, gap = R.select_topk(sb, 4)
    assert ids.tolist() == [[1, 2, 3, 4]] and gap[0] == np.float32(0.3) - np.float32(0.1)
    ids, gap = R.select_topk(sb, 5)
    assert ids.tolist() == [[0, 1, 2, 3, 4]] and np.isinf(gap[0])


def _tiny_route(k=4, bias_shift=0.0, renorm=True, seed=0):
    inp = synth.generate(synth.TINY, seed=seed)
    h = R.rmsnorm(to_f32(inp.x), to_f32(inp.norm_w), 1e-6, round_bf16=False)
    bias = to_f32(inp.bias) + np.float32(bias_shift)
    return h, to_f32(inp.w_router), bias, R.route(h, to_f32(inp.w_router), bias, k, 2.827, renorm)


def test_topk_brute_force_over_all_subsets():
    h, wr, bias, r = _tiny_route()
    sb, ids, gap = r["sb"], r["ids"], r["gap"]
    E, k = sb.shape[1], 4
    subsets = np.array(list(itertools.combinations(range(E), k)))      # 1820 subsets
    sums = sb.astype(np.float64)[:, subsets].sum(axis=2)
    best = subsets[np.argmax(sums, axis=1)]
    checked = 0
    for t in range(sb.shape[0]):
        assert len(set(ids[t])) == k
        if gap[t] > 0:
            assert sorted(best[t]) == list(ids[t])
            checked += 1
    assert checked >= sb.shape[0] - 4


def test_weights_sum_to_routed_scaling():
    _, _, _, r = _tiny_route()
    sums = r["w"].astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(sums, 2.827, rtol=4e-7)
    # ratios follow the unbiased scores
    s_sel = np.take_along_axis(r["s"], r["ids"].astype(np.int64), axis=1).astype(np.float64)
    np.testing.assert_allclose(r["w"] / r["w"][:, :1], s_sel / s_sel[:, :1], rtol=1e-6)


def test_without_renormalisation_weights_are_scaled_scores():
    _, _, _, r = _tiny_route(renorm=False)
    s_sel = np.take_along_axis(r["s"], r["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(r["w"], s_sel * 2.827, rtol=1e-7)


def test_bias_moves_selection_only():
    # a common shift of every bias changes neither the sets nor the weights
    _, _, _, r0 = _tiny_route()
    _, _, _, r1 = _tiny_route(bias_shift=0.25)
    assert np.array_equal(r0["ids"], r1["ids"])
    np.testing.assert_array_equal(r0["w"], r1["w"])
    # a large bias on one expert forces it into every set, weight from its unbiased score
    h, wr, bias, _ = _tiny_route()
    bias = bias.copy()
    bias[5] = 10.0
    r = R.route(h, wr, bias, 4, 2.827, True)
    assert np.all(np.any(r["ids"] == 5, axis=1))
    s_sel = np.take_along_axis(r["s"], r["ids"].astype(np.int64), axis=1).astype(np.float64)
    expect = s_sel / s_sel.sum(axis=1, keepdims=True) * 2.827
    np.testing.assert_allclose(r["w"], expect, rtol=1e-6)


def test_all_experts_selected_when_k_equals_E():
    _, _, _, r = _tiny_route(k=16)
    assert np.all(r["ids"] == np.arange(16)[None, :])


# ------------------------------------------------------------- permutation ---
def _perm_brute(ids, E):
    T, k = ids.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for s in range(k):
                if ids[t, s] == e:
                    rows.append(t * k + s)
    counts = [sum(1 for v in ids.ravel() if v == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return np.array(offsets), np.array(rows)


def test_permutation_brute_force_and_invariants():
    _, _, _, r = _tiny_route()
    ids = r["ids"]
    off, row_pair, pair_row = R.permute(ids, 16)
    boff, brows = _perm_brute(ids, 16)
    assert np.array_equal(off, boff) and np.array_equal(row_pair, brows)
    P = ids.size
    assert off[-1] == P and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(row_pair), np.arange(P))
    assert np.array_equal(pair_row[row_pair], np.arange(P))
    for e in range(16):
        toks = row_pair[off[e]:off[e + 1]] // 4
        assert np.all(np.diff(toks) > 0)
        assert np.all(ids.ravel()[row_pair[off[e]:off[e + 1]]] == e)


# ----------------------------------------------------------------- experts ---
def test_silu_mul_matches_torch():
    rng = np.random.default_rng(5)
    g = rng.normal(0, 4, 4000).astype(np.float32)
    u = rng.normal(0, 1, 4000).astype(np.float32)
    ref = (torch.nn.functional.silu(torch.from_numpy(g).double()) * torch.from_numpy(u).double())
    np.testing.assert_allclose(R.silu_mul(g, u), ref.numpy(), rtol=1e-7, atol=1e-30)


def test_swiglu_gate_and_up_are_not_swapped():
    # token = e_0, so g = Wg[:, 0] = [10, 0] and u = Wu[:, 0] = [-1, 2]
    h = np.zeros((1, 4))
    h[0, 0] = 1.0
    wg = np.zeros((2, 4)); wg[0, 0] = 10.0
    wu = np.zeros((2, 4)); wu[0, 0] = -1.0; wu[1, 0] = 2.0
    wd = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [0.0, 0.0]])
    o, a, _, _ = R.swiglu_expert(h, wg, wu, wd, fp8=False)
    a0 = -10.0 / (1.0 + math.exp(-10.0))        # silu(10) * (-1); silu(0) * 2 = 0
    np.testing.assert_allclose(a[0], [a0, 0.0], rtol=1e-7)
    np.testing.assert_allclose(o[0], [a0, 0.0, a0, 0.0], rtol=1e-7)


def test_swiglu_requantises_before_down_projection():
    # hidden 0 carries amax, hidden 1 a value far below the e4m3 grid of that block
    d, I = 128, 128
    h = np.zeros((1, d)); h[0, 0] = 1.0
    wg = np.zeros((I, d)); wg[0, 0] = 20.0; wg[1, 0] = 20.0
    wu = np.zeros((I, d)); wu[0, 0] = 100.0; wu[1, 0] = 1e-5
    wd = np.zeros((d, I)); wd[0, 0] = 1.0; wd[1, 1] = 1.0
    o8, a, codes, scales = R.swiglu_expert(h, wg, wu, wd, fp8=True)
    o32, _, _, _ = R.swiglu_expert(h, wg, wu, wd, fp8=False)
    assert codes[0, 1] == 0 and o8[0, 1] == 0.0       # below half the smallest subnormal step
    assert o32[0, 1] > 0
    assert codes[0, 0] == 0x7E and o8[0, 0] == np.float32(scales[0, 0] * 448.0)


# ------------------------------------------------------------------- layer ---
def _layer(shape, inp=None, **kw):
    inp = inp if inp is not None else synth.generate(shape, seed=0)
    return inp, run_oracle(inp, **kw)


@pytest.mark.parametrize("fmt", ["f32", "fp8"])
def test_single_expert_reduces_to_dense_swiglu(fmt):
    shape = synth.MoEShape("one", tokens=12, d_model=256, n_experts=1, n_shared=0, top_k=1,
                           d_ff=256, fmt=fmt, routed_scaling=1.0)
    inp, r = _layer(shape)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    x = to_f32(inp.x)
    h = R.rmsnorm(x, to_f32(inp.norm_w), 1e-6, round_bf16=(fmt == "fp8"))
    wts = {k: (None if getattr(inp, k) is None else getattr(inp, k)[0].numpy())
           for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
    if fmt == "fp8":
        q, s = R.quantize_1x128(h)
        hin = R.dequantize_1x128(q, s)
        wg = R.dequantize_weight(wts["w_gate"], wts["s_gate"])
        wu = R.dequantize_weight(wts["w_up"], wts["s_up"])
        wd = R.dequantize_weight(wts["w_down"], wts["s_down"])
    else:
        hin = h.astype(np.float64)
        wg, wu, wd = (wts[k].astype(np.float64) for k in ("w_gate", "w_up", "w_down"))
    g = (hin @ wg.T).astype(np.float32).astype(np.float64)
    u = (hin @ wu.T).astype(np.float32).astype(np.float64)
    a = (g * scipy.special.expit(g) * u).astype(np.float32)
    if fmt == "fp8":
        aq, asc = R.quantize_1x128(a)
        a = R.dequantize_1x128(aq, asc)
    y = (a.astype(np.float64) @ wd.T).astype(np.float32)
    np.testing.assert_allclose(r["y"], y, rtol=2e-6, atol=1e-9)


def test_shared_expert_has_unit_weight():
    shape = synth.MoEShape("one_shared", tokens=8, d_model=256, n_experts=1, n_shared=1,
                           top_k=1, d_ff=128, fmt="f32", routed_scaling=2.5)
    inp = synth.generate(shape, seed=3)
    for name in ("w_gate", "w_up", "w_down"):       # shared expert = routed expert 0
        getattr(inp, name)[1].copy_(getattr(inp, name)[0])
    r = run_oracle(inp)
    np.testing.assert_allclose(r["y"], 3.5 * r["shared"], rtol=2e-6)


def test_sparse_dispatch_equals_dense_masked_formulation():
    shape = synth.small_fp8(tokens=40, n_experts=6, top_k=2)
    inp, r = _layer(shape)
    p = R.params_from_shape(shape)
    hin = R.dequantize_1x128(r["xq"], r["xs"])
    T, E = 40, 6
    wfull = np.zeros((T, E))
    np.put_along_axis(wfull, r["ids"].astype(np.int64), r["w"].astype(np.float64), axis=1)
    y = np.zeros((T, shape.d_model))
    for e in range(E + 1):
        wts = inp.expert_numpy(e)
        wg = R.dequantize_weight(wts["w_gate"], wts["s_gate"])
        wu = R.dequantize_weight(wts["w_up"], wts["s_up"])
        wd = R.dequantize_weight(wts["w_down"], wts["s_down"])
        o, _, _, _ = R.swiglu_expert(hin, wg, wu, wd, True)
        y += (wfull[:, e:e + 1] if e < E else 1.0) * o.astype(np.float64)
    np.testing.assert_allclose(r["y"], y.astype(np.float32), rtol=1e-6, atol=1e-7)
    assert np.array_equal(r["out"], bf16_round((to_f32(inp.x) + r["y"]).astype(np.float32)))


def test_token_permutation_equivariance():
    shape = synth.small_fp8(tokens=24)
    inp = synth.generate(shape, seed=1)
    r0 = run_oracle(inp)
    perm = np.random.default_rng(0).permutation(24)
    inp.x = inp.x[torch.from_numpy(perm)]
    r1 = run_oracle(inp)
    assert np.array_equal(r1["ids"], r0["ids"][perm])
    np.testing.assert_allclose(r1["y"], r0["y"][perm], rtol=1e-6, atol=1e-7)


def test_expert_relabelling_invariance():
    shape = synth.small_fp8(tokens=24, n_experts=8)
    inp = synth.generate(shape, seed=2)
    r0 = run_oracle(inp)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(8))
    full = torch.cat([perm, torch.tensor([8])])
    inp.w_router = inp.w_router[perm]
    inp.bias = inp.bias[perm]
    for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        setattr(inp, name, getattr(inp, name)[full])
    r1 = run_oracle(inp)
    assert np.array_equal(np.sort(perm.numpy()[r1["ids"]], axis=1), r0["ids"])
    np.testing.assert_allclose(r1["y"], r0["y"], rtol=1e-6, atol=1e-7)


def test_doubling_down_scales_doubles_output_exactly():
    shape = synth.small_fp8(tokens=16)
    inp = synth.generate(shape, seed=4)
    r0 = run_oracle(inp)
    inp.s_down = inp.s_down * 2
    r1 = run_oracle(inp)
    assert np.array_equal(r1["y"], r0["y"] * 2)


def test_expert_rows_match_the_layer_per_token():
    """expert_rows (one expert on a subset of tokens) gives, for each token,
    the row the whole layer computes for that (token, expert) pair, and the
    shared expert's output; a token's row does not depend on the others."""
    from oracle.adapt import to_f32
    shape = synth.small_fp8(tokens=20, n_experts=8, top_k=2)
    inp = synth.generate(shape, seed=5)
    r0 = run_oracle(inp)
    p = R.params_from_shape(shape)
    x, g = to_f32(inp.x), to_f32(inp.norm_w)
    for e in range(8):
        ti, si = np.nonzero(r0["ids"] == e)
        if ti.size == 0:
            continue
        o = R.expert_rows(p, x, g, inp.expert_numpy(e), ti)
        assert np.array_equal(o, r0["o_pairs"][ti, si]), e
        # reversed order and a single token give the same rows
        assert np.array_equal(R.expert_rows(p, x, g, inp.expert_numpy(e), ti[::-1]), o[::-1])
        assert np.array_equal(R.expert_rows(p, x, g, inp.expert_numpy(e), ti[-1:]), o[-1:])
    sh = R.expert_rows(p, x, g, inp.expert_numpy(8), np.arange(20))
    assert np.array_equal(sh, r0["shared"])
