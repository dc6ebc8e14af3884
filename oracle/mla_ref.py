"""Plain CPU definition of Kimi K2's multi-head latent attention (MLA) sub-layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages define it:

* block dataflow -- "Kimi K2 · Dense transformer block", Code: the attention
  half of a block is residual = h; h = input_layernorm(h); h = self_attn(h);
  h = residual + h.  The sub-layer here is that half: out = x + MLA(RMSNorm(x)).
* shape -- "Kimi K2 · Architecture", Fact sheet (Attention: 64 heads; keys
  128 + 64 rotary features, values 128; latents: query 1,536, key-value 512)
  and config.json (num_attention_heads 64, q_lora_rank 1536, kv_lora_rank
  512, qk_nope_head_dim 128, qk_rope_head_dim 64, v_head_dim 128,
  attention_bias false, rms_norm_eps 1e-6).
* latent norms -- "Kimi-K2-Base", Attention, QK norm: RMSNorm only on the
  query and key-value latents, before their up-projections; no per-head norm.
* positional key -- "Kimi-K2-Base", Attention: partial RoPE on 64 of the 192
  query/key features; one 64-wide positional key shared by all heads and
  cached next to the 512-wide latent (Decoupled RoPE dim).
* RoPE base and YaRN -- config.json rope_theta 50000 and rope_scaling (yarn,
  factor 32, original_max_position_embeddings 4096, beta_fast = beta_slow =
  1, mscale = mscale_all_dim = 1); the softmax scale is 1/sqrt(192) times
  the square of the YaRN attention correction 0.1 ln(32) + 1 ("Kimi K2 ·
  Architecture", the YaRN RoPE source note; "Kimi-K2-Base", Context).
* scores -- "Kimi-K2-Base", Attention: the query-key product times the
  softmax scale; causal mask; positions numbered from the cached length
  ("Kimi K2 · Architecture", the model source note).
* FP8 -- config.json quantization_config: every projection matrix is e4m3
  with 128x128 block scales and dynamically quantised activations
  ("Kimi K2 · Dense transformer block", Weights: Attention, FP8).

Readings where the pages are silent (listed in the design notes): the RoPE
pairs are consecutive features (2i, 2i+1) rotated by position * f_i; YaRN
keeps the base frequency of pair i when the original context holds more than
beta_fast turns of it and divides it by the factor when it holds fewer than
beta_slow turns (the two betas are equal here, so the ramp between them is a
step); the rotary magnitude correction mscale / mscale_all_dim is 1; per head
the query is [128 no-position features, 64 rotary], the key-value
up-projection gives [128 key features, 128 value features]; every FP8 linear
quantises its input per 1x128 (so the cached latent is held as its e4m3
codes and scales, which is exactly what the key-value up-projection reads);
normalised latents and h are rounded to bf16, the rotary key to bf16 (the
cache), everything else is fp32; scores, softmax and the value sum are exact
sums rounded to fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .fp8 import bf16_round, e4m3_decode, f32
from .moe_ref import BLOCK, dequantize_1x128, quantize_1x128, rmsnorm


@dataclass(frozen=True)
class MLAParams:
    d_model: int = 7168
    n_heads: int = 64
    q_lora: int = 1536
    kv_lora: int = 512
    qk_nope: int = 128
    qk_rope: int = 64
    v_head: int = 128
    rope_theta: float = 50000.0
    rope_factor: float = 32.0
    rope_orig_len: int = 4096
    beta_fast: float = 1.0
    beta_slow: float = 1.0
    mscale_all_dim: float = 1.0
    rms_eps: float = 1e-6

    @property
    def q_head(self) -> int:
        return self.qk_nope + self.qk_rope


def weight_shapes(p: MLAParams) -> dict:
    """nn.Linear [out, in] shape of every projection and the two latent norms."""
    return {
        "w_qa": (p.q_lora, p.d_model),
        "w_qb": (p.n_heads * p.q_head, p.q_lora),
        "w_kva": (p.kv_lora + p.qk_rope, p.d_model),
        "w_kvb": (p.n_heads * (p.qk_nope + p.v_head), p.kv_lora),
        "w_o": (p.d_model, p.n_heads * p.v_head),
        "g_qa": (p.q_lora,),
        "g_kva": (p.kv_lora,),
    }


def param_count(p: MLAParams) -> int:
    return int(sum(np.prod(s) for s in weight_shapes(p).values()))


# ---------------------------------------------------------------- YaRN RoPE
def yarn_inv_freq(p: MLAParams) -> np.ndarray:
    """Per rotary pair i: f_i = base^(-2i/dim), kept when the original context
    spans more than beta_fast turns of it (high frequency), divided by the
    factor when it spans fewer than beta_slow turns (low frequency), and
    linearly blended in between (float64)."""
    dim = p.qk_rope
    i = np.arange(dim // 2, dtype=np.float64)
    f = p.rope_theta ** (-2.0 * i / dim)
    turns = p.rope_orig_len * f / (2.0 * math.pi)       # turns over the original context
    if p.beta_fast == p.beta_slow:
        keep = (turns > p.beta_fast).astype(np.float64)
    else:
        keep = np.clip((turns - p.beta_slow) / (p.beta_fast - p.beta_slow), 0.0, 1.0)
    return keep * f + (1.0 - keep) * f / p.rope_factor


def softmax_scale(p: MLAParams) -> float:
    corr = 0.1 * p.mscale_all_dim * math.log(p.rope_factor) + 1.0
    return corr * corr / math.sqrt(p.q_head)


def apply_rope(v: np.ndarray, pos: np.ndarray, p: MLAParams) -> np.ndarray:
    """Rotate the consecutive feature pairs (2i, 2i+1) of v [..., n, dim] by
    pos[n] * f_i (float64 in, float64 out)."""
    ang = pos.astype(np.float64)[:, None] * yarn_inv_freq(p)[None, :]     # [n, dim/2]
    c, s = np.cos(ang), np.sin(ang)
    v = v.astype(np.float64)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ------------------------------------------------------------- FP8 linears
def dequantize_weight_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N, K] codes with [ceil(N/128), K/128] block scales -> float64 (exact).
    The last row block may be partial (the 576-row key-value down-projection)."""
    N, K = codes.shape
    vals = e4m3_decode(codes).reshape(N, K // BLOCK, BLOCK)
    rb = np.arange(N) // BLOCK
    vals = vals * scales.astype(np.float64)[rb][:, :, None]
    return vals.reshape(N, K)


def fp8_linear(a: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y = dq(q(a)) . dq(W)^T: input quantised per 1x128, exact sum rounded to fp32."""
    q, s = quantize_1x128(a)
    return f32(dequantize_1x128(q, s) @ dequantize_weight_rows(codes, scales).T)


# ------------------------------------------------------------------ layer
def latents(p: MLAParams, x: np.ndarray, w: dict):
    """Projections of the new tokens up to the cache entries.

    Returns h (bf16 values), q [T, heads, 192] fp32 with the rotary part not
    yet rotated, the normalised key-value latent c (bf16 values) and the
    unrotated positional key kpe [T, 64] fp32."""
    h = rmsnorm(x, w["g_in"], p.rms_eps, round_bf16=True)
    qa = fp8_linear(h, w["w_qa"], w["s_qa"])
    qa_n = rmsnorm(qa, w["g_qa"], p.rms_eps, round_bf16=True)
    q = fp8_linear(qa_n, w["w_qb"], w["s_qb"]).reshape(-1, p.n_heads, p.q_head)
    kva = fp8_linear(h, w["w_kva"], w["s_kva"])
    c = rmsnorm(kva[:, :p.kv_lora], w["g_kva"], p.rms_eps, round_bf16=True)
    kpe = kva[:, p.kv_lora:]
    return h, q, c, kpe


def cache_entries(p: MLAParams, c: np.ndarray, kpe: np.ndarray, pos: np.ndarray):
    """What one position stores: the e4m3 codes and 1x128 scales of the
    latent (the input of the key-value up-projection) and the rotated
    positional key rounded to bf16."""
    codes, scales = quantize_1x128(c)
    k_rot = bf16_round(f32(apply_rope(kpe, pos, p)))
    return codes, scales, k_rot


def attend(p: MLAParams, q: np.ndarray, qpos: int, keys_codes: np.ndarray,
           keys_scales: np.ndarray, keys_rope: np.ndarray, w: dict) -> np.ndarray:
    """One query token over cache positions 0..qpos (causal).

    q [heads, 192] fp32 (rotary part unrotated); keys_* hold positions
    0..L-1 (L > qpos).  Per head: k = [W_uk c_j, kpe_j], v = W_uv c_j with c_j
    the dequantised cached latent; s_j = scale (q . k_j); p = softmax(s);
    o = sum_j p_j v_j.  Returns o [heads * 128] fp32."""
    n = qpos + 1
    H, dn, dr, dv = p.n_heads, p.qk_nope, p.qk_rope, p.v_head
    c = dequantize_1x128(keys_codes[:n], keys_scales[:n])                 # [n, 512] float64
    wkvb = dequantize_weight_rows(w["w_kvb"], w["s_kvb"])                 # [H*(dn+dv), 512]
    kv = f32(wkvb @ c.T).reshape(H, dn + dv, n).astype(np.float64)       # up-projection
    k_nope, v = kv[:, :dn, :], kv[:, dn:, :]                              # [H, 128, n] each
    q_nope = q[:, :dn].astype(np.float64)
    q_rot = apply_rope(q[:, dn:][None], np.array([qpos]), p)[0]          # [H, 64]
    s = np.einsum("hd,hdn->hn", q_nope, k_nope) + q_rot @ keys_rope[:n].astype(np.float64).T
    s = f32(s * softmax_scale(p))
    s64 = s.astype(np.float64)
    e = np.exp(s64 - s64.max(axis=1, keepdims=True))
    pr = f32(e / e.sum(axis=1, keepdims=True))
    o = f32(np.einsum("hn,hdn->hd", pr.astype(np.float64), v))
    return o.reshape(H * dv)


def mla_layer(p: MLAParams, x: np.ndarray, w: dict, seq_of: np.ndarray, pos_of: np.ndarray,
              cache: dict, tokens=None) -> dict:
    """The attention half of a block for T new tokens: out = x + o_proj(MLA(RMSNorm(x))).

    x [T, d] (bf16 values as fp32); seq_of[t], pos_of[t]: the token's
    sequence and position (its sequence's cached length plus its index among
    that sequence's new tokens).  cache: dict of "codes" [S, L, 512] u8,
    "scales" [S, L, 4] fp32, "rope" [S, L, 64] fp32 (bf16 values) holding
    positions below each sequence's cached length; the new tokens' entries
    are written into it (in place) before any token attends.  Outputs are
    computed for ``tokens`` (default all).  Returns the new cache entries and
    o (attention output before o_proj), y and out of the selected tokens."""
    T = x.shape[0]
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    h, q, c, kpe = latents(p, x, w)
    codes, scales, k_rot = cache_entries(p, c, kpe, pos_of)
    cache["codes"][seq_of, pos_of] = codes
    cache["scales"][seq_of, pos_of] = scales
    cache["rope"][seq_of, pos_of] = k_rot
    o = np.zeros((len(sel), p.n_heads * p.v_head), dtype=np.float32)
    for i, t in enumerate(sel):
        s_ = int(seq_of[t])
        o[i] = attend(p, q[t], int(pos_of[t]), cache["codes"][s_], cache["scales"][s_],
                      cache["rope"][s_], w)
    y = fp8_linear(o, w["w_o"], w["s_o"])
    out = bf16_round(f32(f32(x[sel]) + y))
    return dict(h=h, q=q, c=c, kpe=kpe, codes=codes, scales=scales, k_rot=k_rot,
                tokens=sel, o=o, y=y, out=out)
