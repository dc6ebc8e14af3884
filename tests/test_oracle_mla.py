"""Pins of the MLA attention oracle (oracle/mla_ref.py) against what the pages
and the mathematics fix.  CPU only."""
import math

import numpy as np
import pytest

from oracle import mla_ref as M
from oracle.fp8 import bf16_round, f32
from oracle.moe_ref import quantize_1x128

K2 = M.MLAParams()
# a small MLA with the same structure: every FP8 linear's input width a
# multiple of 128, the rotary width even
TINY = M.MLAParams(d_model=256, n_heads=2, q_lora=128, kv_lora=128, qk_nope=16, qk_rope=8,
                   v_head=64)


def test_parameter_count_matches_the_page():
    """"Kimi K2 · Dense transformer block", Parameters: multi-head latent
    attention 101,124,096 (q_a 7168x1536, q_b 1536x(64x192), kv_a 7168x576,
    kv_b 512x(64x256), o 8192x7168 and the two latent norms)."""
    assert M.param_count(K2) == 101_124_096


def test_cache_bytes_per_token():
    """"Kimi-K2-Base", KV cache: 70,272 B per token = 61 layers x (512 + 64)
    16-bit entries; the FP8 latent layout holds 512 codes, four fp32 scales
    and the 64 bf16 rotary features."""
    assert 61 * (K2.kv_lora + K2.qk_rope) * 2 == 70_272
    assert K2.kv_lora + 4 * (K2.kv_lora // 128) + 2 * K2.qk_rope == 656


def test_softmax_scale_closed_form():
    """1/sqrt(192) x (0.1 ln 32 + 1)^2 ("Kimi-K2-Base", Context: the YaRN
    release note)."""
    assert M.softmax_scale(K2) == pytest.approx(0.13086079996295008, rel=1e-15)
    assert M.softmax_scale(M.MLAParams(rope_factor=1.0)) == pytest.approx(1 / math.sqrt(192))


def test_yarn_reduces_to_rope_without_scaling():
    p = M.MLAParams(rope_factor=1.0)
    i = np.arange(32)
    np.testing.assert_allclose(M.yarn_inv_freq(p), 50000.0 ** (-i / 32.0), rtol=1e-15)


def test_yarn_k2_frequencies():
    """With beta_fast = beta_slow = 1 a pair keeps its base frequency when the
    4096-position original context spans more than one turn of it: pair 19
    spans 1.057 turns (4096 * 50000^(-38/64) / 2 pi), pair 20 spans 0.754, so
    pairs 0..19 keep f_i and pairs 20..31 take f_i / 32."""
    f = 50000.0 ** (-np.arange(32) / 32.0)
    got = M.yarn_inv_freq(K2)
    np.testing.assert_array_equal(got[:20], f[:20])
    np.testing.assert_allclose(got[20:], f[20:] / 32.0, rtol=1e-15)
    # a ramp between distinct betas is linear in the number of turns
    p = M.MLAParams(beta_fast=32.0, beta_slow=1.0)
    turns = 4096 * f / (2 * math.pi)
    keep = np.clip((turns - 1.0) / 31.0, 0, 1)
    np.testing.assert_allclose(M.yarn_inv_freq(p), keep * f + (1 - keep) * f / 32, rtol=1e-14)


def test_rope_is_a_rotation_with_relative_positions():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((5, 64))
    k = rng.standard_normal((5, 64))
    m = np.array([0, 3, 17, 4095, 70000])
    n = np.array([2, 3, 1, 9, 131071])
    rq, rk = M.apply_rope(q, m, K2), M.apply_rope(k, n, K2)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(M.apply_rope(q[:1], np.array([0]), K2), q[:1])
    s = 37
    rq2, rk2 = M.apply_rope(q, m + s, K2), M.apply_rope(k, n + s, K2)
    np.testing.assert_allclose(np.sum(rq * rk, axis=1), np.sum(rq2 * rk2, axis=1),
                               rtol=1e-9, atol=1e-9)
    # pair 0 of a unit vector turns by exactly the position (frequency 1)
    e = np.zeros((1, 64))
    e[0, 0] = 1.0
    r = M.apply_rope(e, np.array([1]), K2)
    assert r[0, 0] == pytest.approx(math.cos(1.0)) and r[0, 1] == pytest.approx(math.sin(1.0))


def _tiny_weights(p, seed=0):
    from synth.gen import block_quantize_weight
    import torch
    rng = np.random.default_rng(seed)
    w = {}
    for name, shp in M.weight_shapes(p).items():
        if name.startswith("g_"):
            w[name] = bf16_round(f32(1.0 + 0.1 * rng.standard_normal(shp)))
            continue
        n, k = shp
        npad = (n + 127) // 128 * 128
        full = rng.standard_normal((npad, k)).astype(np.float32) * 0.02
        codes, scales = block_quantize_weight(torch.from_numpy(full))
        w[name] = codes.numpy()[:n]
        w["s" + name[1:]] = scales.numpy()
    w["g_in"] = bf16_round(f32(1.0 + 0.1 * rng.standard_normal(p.d_model)))
    return w


def _empty_cache(p, S, L):
    return dict(codes=np.zeros((S, L, p.kv_lora), np.uint8),
                scales=np.ones((S, L, p.kv_lora // 128), np.float32),
                rope=np.zeros((S, L, p.qk_rope), np.float32))


def test_partial_row_block_dequantisation():
    """The 576-row key-value down-projection has a last row block of 64 rows:
    row r takes scale block r // 128."""
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7E, size=(192, 256)).astype(np.uint8)
    scales = rng.random((2, 2)).astype(np.float32) + 0.5
    from oracle.fp8 import e4m3_decode
    want = e4m3_decode(codes) * np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)[:192]
    np.testing.assert_array_equal(M.dequantize_weight_rows(codes, scales), want)


def _brute_attend(p, q, qpos, codes, scales, rope, w):
    """Scalar loops over heads, positions and features (tiny sizes only)."""
    from oracle.fp8 import e4m3_decode
    H, dn, dr, dv, R = p.n_heads, p.qk_nope, p.qk_rope, p.v_head, p.kv_lora
    kvb = e4m3_decode(w["w_kvb"]).astype(np.float64)
    sk = w["s_kvb"].astype(np.float64)
    f = M.yarn_inv_freq(p)
    scale = M.softmax_scale(p)
    out = []
    for h in range(H):
        qr = []
        for i in range(dr // 2):
            a, b = float(q[h, dn + 2 * i]), float(q[h, dn + 2 * i + 1])
            c, s = math.cos(qpos * f[i]), math.sin(qpos * f[i])
            qr += [a * c - b * s, a * s + b * c]
        scores, vals = [], []
        for j in range(qpos + 1):
            lat = [float(e4m3_decode(np.array([codes[j, r]]))[0]) * float(scales[j, r // 128])
                   for r in range(R)]
            k = []
            for o in range(dn + dv):
                row = h * (dn + dv) + o
                k.append(float(f32(sum(kvb[row, r] * sk[row // 128, r // 128] * lat[r]
                                       for r in range(R)))))
            dot = sum(float(q[h, d]) * k[d] for d in range(dn))
            dot += sum(qr[d] * float(rope[j, d]) for d in range(dr))
            scores.append(float(f32(dot * scale)))
            vals.append(k[dn:])
        mx = max(scores)
        e = [math.exp(s_ - mx) for s_ in scores]
        z = sum(e)
        pr = [float(f32(x / z)) for x in e]
        out += [sum(pr[j] * vals[j][d] for j in range(qpos + 1)) for d in range(dv)]
    return np.array(out)


def test_attention_matches_scalar_loops():
    p = TINY
    w = _tiny_weights(p, seed=2)
    rng = np.random.default_rng(3)
    L = 5
    c = bf16_round(f32(rng.standard_normal((L, p.kv_lora))))
    codes, scales = quantize_1x128(c)
    rope = bf16_round(f32(rng.standard_normal((L, p.qk_rope))))
    q = f32(rng.standard_normal((p.n_heads, p.q_head)))
    for qpos in (0, 2, 4):
        got = M.attend(p, q, qpos, codes, scales, rope, w)
        want = _brute_attend(p, q, qpos, codes, scales, rope, w)
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=1e-7)


def test_attention_special_cases():
    p = TINY
    w = _tiny_weights(p, seed=4)
    rng = np.random.default_rng(5)
    L = 6
    c = bf16_round(f32(rng.standard_normal((L, p.kv_lora))))
    codes, scales = quantize_1x128(c)
    rope = bf16_round(f32(rng.standard_normal((L, p.qk_rope))))
    q = f32(rng.standard_normal((p.n_heads, p.q_head)))
    wkvb = M.dequantize_weight_rows(w["w_kvb"], w["s_kvb"]).reshape(
        p.n_heads, p.qk_nope + p.v_head, p.kv_lora)
    from oracle.moe_ref import dequantize_1x128
    lat = dequantize_1x128(codes, scales)
    v = f32(np.einsum("hok,nk->hno", wkvb, lat))[:, :, p.qk_nope:]
    # one visible position: the output is that position's value
    np.testing.assert_allclose(M.attend(p, q, 0, codes, scales, rope, w),
                               v[:, 0].reshape(-1), rtol=1e-6)
    # a zero query weighs every visible position equally
    o = M.attend(p, np.zeros_like(q), 3, codes, scales, rope, w)
    np.testing.assert_allclose(o, v[:, :4].mean(axis=1).reshape(-1), rtol=1e-5, atol=1e-7)
    # causal: positions after the query do not matter
    codes2, rope2 = codes.copy(), rope.copy()
    codes2[4:] = 0x38
    rope2[4:] = 7.0
    np.testing.assert_array_equal(M.attend(p, q, 3, codes, scales, rope, w),
                                  M.attend(p, q, 3, codes2, scales, rope2, w))


def test_prefill_equals_token_by_token_decode():
    """All new tokens of a sequence at once (their entries written first, each
    attending up to its own position) give exactly what feeding them one at a
    time through the cache gives; a second sequence is independent."""
    p = TINY
    w = _tiny_weights(p, seed=6)
    rng = np.random.default_rng(7)
    T = 5
    x = bf16_round(f32(rng.standard_normal((T, p.d_model))))
    seq = np.zeros(T, np.int64)
    pos = np.arange(T)
    ca = _empty_cache(p, 2, 8)
    ra = M.mla_layer(p, x, w, seq, pos, ca)
    cb = _empty_cache(p, 2, 8)
    outs = [M.mla_layer(p, x[t:t + 1], w, seq[t:t + 1], pos[t:t + 1], cb)["out"][0]
            for t in range(T)]
    np.testing.assert_array_equal(ra["out"], np.stack(outs))
    for k in ("codes", "scales", "rope"):
        np.testing.assert_array_equal(ca[k], cb[k])
    # the same tokens as sequence 1 continuing after 2 cached positions: only
    # their positions change the result, and sequence 0's entries are untouched
    cc = _empty_cache(p, 2, 8)
    cc["codes"][1, :2], cc["scales"][1, :2], cc["rope"][1, :2] = ca["codes"][0, :2], \
        ca["scales"][0, :2], ca["rope"][0, :2]
    r1 = M.mla_layer(p, x[2:], w, np.ones(3, np.int64), pos[2:], cc)
    np.testing.assert_array_equal(r1["out"], ra["out"][2:])
    assert not cc["codes"][0].any()


def test_layer_without_attention_mixing_is_the_projection_chain():
    """Zero key-value up-projection scales: every value is 0, so the attention
    output is 0 and the layer returns x rounded (residual only); o_proj of a
    zero input is 0."""
    p = TINY
    w = _tiny_weights(p, seed=8)
    w["s_kvb"] = np.zeros_like(w["s_kvb"])
    rng = np.random.default_rng(9)
    x = bf16_round(f32(rng.standard_normal((3, p.d_model))))
    r = M.mla_layer(p, x, w, np.zeros(3, np.int64), np.arange(3), _empty_cache(p, 1, 4))
    assert not r["o"].any() and not r["y"].any()
    np.testing.assert_array_equal(r["out"], x)
