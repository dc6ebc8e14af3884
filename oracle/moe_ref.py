"""Plain CPU definition of one Kimi K2 MoE feed-forward sub-layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, step by step, and where the pages define it:

* block dataflow -- "Kimi K2 · Dense transformer block", Code: the FFN half
  of a block is residual = h; h = post_attention_layernorm(h); h = mlp(h);
  h = residual + h.  The layer here is that half: out = x + FFN(RMSNorm(x)).
* RMSNorm, eps 1e-6 -- "Kimi-K2-Base", Normalization and stability (RMSNorm,
  pre-norm, eps 1e-06); config.json rms_norm_eps.
* router -- "Kimi-K2-Base", Mixture of experts: sigmoid router score; the
  correction bias is added to the sigmoid scores for top-k selection only
  (Load balancing, the scores_for_choice line); one expert group
  (Group-limited routing: none, n_group = topk_group = 1); 8 of 384 experts
  (Experts per token); the selected weights are renormalised to sum to 1
  (Renormalize top-k) and then multiplied by 2.827 (Routed scaling factor).
* experts -- "Kimi-K2-Base", Feed-forward, Activation:
  down_proj(act_fn(gate_proj(x)) * up_proj(x)) with act_fn = SiLU and no
  biases (FFN bias: No); 2048 hidden features per expert, one shared expert
  applied to every token ("Kimi K2 · Architecture", Fact sheet, Feed-forward).
* FP8 -- "Kimi K2 · Architecture", config.json quantization_config: fp8,
  e4m3, 128x128 weight blocks, dynamic activations; "Kimi-K2-Base",
  Pretraining recipe, Training precision: FP8-E4M3 in 1x128 tiles with fp32
  scales (taken as the activation granularity).

Readings where the pages are silent are listed in the design notes; the ones
that change a number here are: scale = amax/448 with a zero block giving
scale 1 and codes 0; q = e4m3(clamp(h/scale)) with IEEE fp32 division; the
SwiGLU output is requantised per 1x128 before the down projection; the
shared expert has weight 1; top-k ties go to the lower expert id; ids are
stored ascending; combine order is ascending expert id, shared expert last.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from .fp8 import E4M3_MAX, bf16_round, e4m3_decode, e4m3_encode, f32

BLOCK = 128


@dataclass(frozen=True)
class LayerParams:
    d_model: int
    n_experts: int
    n_shared: int
    top_k: int
    d_ff: int
    fp8: bool
    routed_scaling: float = 2.827
    rms_eps: float = 1e-6
    norm_topk_prob: bool = True
    dense: bool = False


# ---------------------------------------------------------------- RMSNorm ---
def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, round_bf16: bool) -> np.ndarray:
    """h = x / sqrt(mean(x^2) + eps) * gamma.

    mean(x^2) is the exact mean rounded to fp32; r = 1/sqrt(ms + eps) uses
    fp32 IEEE add, sqrt and divide; h = (x * r) * gamma in fp32, then one
    rounding to bf16 for the bf16 layer.
    """
    x = f32(x)
    ms = f32(np.mean(x.astype(np.float64) ** 2, axis=1))
    r = f32(np.float32(1.0) / np.sqrt(ms + np.float32(eps)))
    h = f32(f32(x * r[:, None]) * f32(gamma)[None, :])
    return bf16_round(h) if round_bf16 else h


# ------------------------------------------------ 1x128 activation quant ---
def quantize_1x128(a: np.ndarray):
    """Dynamic per-row, per-128-column FP8 quantisation.

    scale = amax/448 (fp32 divide); a zero block takes scale 1;
    code = e4m3(clamp(a/scale, -448, 448)) with fp32 division.
    Returns (codes uint8 [R, C], scales fp32 [R, C/128]).
    """
    a = f32(a)
    R, C = a.shape
    assert C % BLOCK == 0
    blk = a.reshape(R, C // BLOCK, BLOCK)
    amax = f32(np.max(np.abs(blk), axis=2))
    scale = f32(amax / np.float32(E4M3_MAX))
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    v = f32(blk / scale[:, :, None])
    v = np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = e4m3_encode(v).reshape(R, C)
    return codes, scale


def dequantize_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [R, C], scales [R, C/128] -> float64 values (exact)."""
    R, C = codes.shape
    vals = e4m3_decode(codes).reshape(R, C // BLOCK, BLOCK)
    return (vals * scales.astype(np.float64)[:, :, None]).reshape(R, C)


def dequantize_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N, K] codes with [N/128, K/128] block scales -> float64 [N, K] (exact)."""
    N, K = codes.shape
    vals = e4m3_decode(codes).reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    vals *= scales.astype(np.float64)[:, None, :, None]
    return vals.reshape(N, K)


# ----------------------------------------------------------------- router ---
def router_logits(h: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z = h . W_r^T, exact products and sum, rounded to fp32."""
    return f32(h.astype(np.float64) @ w_router.astype(np.float64).T)


def sigmoid_scores(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)), rounded to fp32."""
    return f32(1.0 / (1.0 + np.exp(-z.astype(np.float64))))


def select_topk(sb: np.ndarray, k: int):
    """Top-k of the biased scores, one group, ties to the lower expert id.

    Returns ids [T, k] ascending and gap [T] = sb_(k) - sb_(k+1) (fp32;
    +inf when every expert is selected).
    """
    T, E = sb.shape
    order = np.argsort(-sb, axis=1, kind="stable")      # stable: equal keys keep ascending id
    ids = np.sort(order[:, :k], axis=1).astype(np.int32)
    rows = np.arange(T)
    if k < E:
        gap = f32(sb[rows, order[:, k - 1]] - sb[rows, order[:, k]])
    else:
        gap = np.full(T, np.inf, dtype=np.float32)
    return ids, gap


def routing_weights(s: np.ndarray, ids: np.ndarray, scaling: float, renorm: bool) -> np.ndarray:
    """Weights from the unbiased scores of the chosen experts.

    renormalise (divide by their exact sum, rounded to fp32), then multiply
    by the routed scaling factor, both in fp32.
    """
    ssel = f32(np.take_along_axis(s, ids.astype(np.int64), axis=1))
    if renorm:
        denom = f32(np.sum(ssel.astype(np.float64), axis=1))
        w = f32(ssel / denom[:, None])
    else:
        w = ssel
    return f32(w * np.float32(scaling))


def route(h, w_router, bias, k, scaling, renorm):
    z = router_logits(h, w_router)
    s = sigmoid_scores(z)
    sb = f32(s + f32(bias)[None, :])
    ids, gap = select_topk(sb, k)
    w = routing_weights(s, ids, scaling, renorm)
    return dict(z=z, s=s, sb=sb, ids=ids, gap=gap, w=w)


# ------------------------------------------------------------ permutation ---
def permute(ids: np.ndarray, n_experts: int):
    """Group the (token, slot) pairs by expert, tokens ascending within one.

    offsets [E+1] is the exclusive prefix sum of the per-expert counts;
    row_pair[row] = t*k + slot; pair_row is its inverse.
    """
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_pair = np.argsort(flat, kind="stable").astype(np.int32)   # pair index order = token order
    pair_row = np.empty_like(row_pair)
    pair_row[row_pair] = np.arange(flat.size, dtype=np.int32)
    return offsets, row_pair, pair_row


# ---------------------------------------------------------------- experts ---
def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """a = silu(g) * u = g / (1 + exp(-g)) * u, rounded to fp32."""
    g64 = g.astype(np.float64)
    return f32(g64 / (1.0 + np.exp(-g64)) * u.astype(np.float64))


def swiglu_expert(hrows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                  fp8: bool):
    """One SwiGLU expert on rows of (dequantised) activations.

    hrows: float64 [m, d] (already dequantised in the FP8 layer);
    wg, wu: float64 [I, d]; wd: float64 [d, I] (dequantised weights).
    g and u are exact dot products rounded to fp32; in the FP8 layer the
    SwiGLU output is requantised per 1x128 before the down projection.
    Returns (o fp32 [m, d], a fp32 [m, I], a_codes, a_scales).
    """
    g = f32(hrows @ wg.T)
    u = f32(hrows @ wu.T)
    a = silu_mul(g, u)
    if fp8:
        a_codes, a_scales = quantize_1x128(a)
        o = down_projection(a_codes, a_scales, wd)
    else:
        a_codes = a_scales = None
        o = f32(a.astype(np.float64) @ wd.T)
    return o, a, a_codes, a_scales


def down_projection(a_codes: np.ndarray, a_scales: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """o = dequant(a) . W_down^T from requantised SwiGLU activations (exact, to fp32)."""
    return f32(dequantize_1x128(a_codes, a_scales) @ wd.T)


# ----------------------------------------------------------------- layer ---
def _expert_f64(wts: dict, fp8: bool):
    if fp8:
        return (dequantize_weight(wts["w_gate"], wts["s_gate"]),
                dequantize_weight(wts["w_up"], wts["s_up"]),
                dequantize_weight(wts["w_down"], wts["s_down"]))
    return (wts["w_gate"].astype(np.float64), wts["w_up"].astype(np.float64),
            wts["w_down"].astype(np.float64))


def moe_layer(p: LayerParams, x: np.ndarray, norm_w: np.ndarray,
              w_router: Optional[np.ndarray], bias: Optional[np.ndarray],
              expert: Callable[[int], dict], tokens: Optional[np.ndarray] = None) -> dict:
    """Full sub-layer: out = x + MoE(RMSNorm(x)).

    x, norm_w, w_router: float32 arrays holding the (exact) values of the
    bf16 / fp32 inputs; bias fp32.  expert(e) returns one expert's weights
    (codes + scales, or fp32), e = n_experts .. n_experts+n_shared-1 being
    the shared experts.  Routing and the permutation cover every token;
    expert outputs, y and out are computed for ``tokens`` (default: all).
    """
    T = x.shape[0]
    k, E = p.top_k, p.n_experts
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    res: dict = {}

    h = rmsnorm(x, norm_w, p.rms_eps, round_bf16=p.fp8)
    res["h"] = h
    if p.dense:
        ids = np.zeros((T, 1), dtype=np.int32)
        w = np.ones((T, 1), dtype=np.float32) * np.float32(p.routed_scaling)
        res.update(ids=ids, w=w, gap=np.full(T, np.inf, np.float32))
    else:
        res.update(route(h, w_router, bias, k, p.routed_scaling, p.norm_topk_prob))
    offsets, row_pair, pair_row = permute(res["ids"], E)
    res.update(offsets=offsets, row_pair=row_pair, pair_row=pair_row)

    hs = h[sel]
    if p.fp8:
        xq, xs = quantize_1x128(hs)
        hin = dequantize_1x128(xq, xs)
        res.update(xq=xq, xs=xs)
    else:
        hin = hs.astype(np.float64)

    used = res["ids"][sel]
    wsel = res["w"][sel]
    n = len(sel)
    kk = used.shape[1]
    o_pairs = np.zeros((n, kk, p.d_model), dtype=np.float32)
    a_pairs = np.zeros((n, kk, p.d_ff), dtype=np.float32)
    for e in np.unique(used):
        ti, si = np.nonzero(used == e)
        wg, wu, wd = _expert_f64(expert(int(e)), p.fp8)
        o, a, _, _ = swiglu_expert(hin[ti], wg, wu, wd, p.fp8)
        o_pairs[ti, si] = o
        a_pairs[ti, si] = a
        del wg, wu, wd
    shared_parts = []
    for j in range(p.n_shared):
        wg, wu, wd = _expert_f64(expert(E + j), p.fp8)
        o, _, _, _ = swiglu_expert(hin, wg, wu, wd, p.fp8)
        shared_parts.append(o)
        del wg, wu, wd

    # y = sum over the token's experts in ascending id of w * o, then the
    # shared expert(s) with weight 1; out = x + y rounded once
    y64 = np.einsum("ts,tsd->td", wsel.astype(np.float64), o_pairs.astype(np.float64))
    for o in shared_parts:
        y64 = y64 + o.astype(np.float64)
    shared = (f32(np.sum([o.astype(np.float64) for o in shared_parts], axis=0)) if shared_parts
              else np.zeros((n, p.d_model), dtype=np.float32))
    y = f32(y64)
    out = f32(f32(x[sel]) + y)
    out = bf16_round(out) if p.fp8 else out
    res.update(tokens=sel, o_pairs=o_pairs, a_pairs=a_pairs, shared=shared, y=y, out=out)
    return res


def expert_rows(p: LayerParams, x: np.ndarray, norm_w: np.ndarray, wts: dict,
                tokens: np.ndarray) -> np.ndarray:
    """One expert's unweighted output o for the given tokens (fp32 [n, d]).

    The same steps as the layer for those tokens alone: RMSNorm, activation
    quantisation (FP8 layer), then the SwiGLU expert.  Each token's row
    depends only on that token, so any subset of an expert's tokens can be
    checked without running the rest of the layer.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    h = rmsnorm(x[tokens], norm_w, p.rms_eps, round_bf16=p.fp8)
    if p.fp8:
        xq, xs = quantize_1x128(h)
        hin = dequantize_1x128(xq, xs)
    else:
        hin = h.astype(np.float64)
    wg, wu, wd = _expert_f64(wts, p.fp8)
    o, _, _, _ = swiglu_expert(hin, wg, wu, wd, p.fp8)
    return o


def params_from_shape(shape) -> LayerParams:
    return LayerParams(d_model=shape.d_model, n_experts=shape.n_experts, n_shared=shape.n_shared,
                       top_k=shape.top_k, d_ff=shape.d_ff, fp8=(shape.fmt == "fp8"),
                       routed_scaling=shape.routed_scaling, rms_eps=shape.rms_eps,
                       norm_topk_prob=shape.norm_topk_prob, dense=shape.dense)
