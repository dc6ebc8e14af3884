"""CPU oracle of one training step of the MoE layer: the forward in BF16
compute that keeps FP8 copies of the up-projection and SwiGLU inputs, and
the backward that reads those copies.

Test infrastructure only: imported by tests/, the smoke check and the CPU
baseline of bench.py, never by the product path.

What the pages fix ("Kimi-K2-Base", Pretraining recipe, Training precision):
no FP8 in computation; the inputs of the MoE up-projections and of SwiGLU
are compressed to FP8-E4M3 in 1x128 tiles with FP32 scales for the backward.
Readings taken where the pages stop:

* the layer is the FFN half of a block, out = x + MoE(RMSNorm(x)), with bf16
  weights (router, experts, the norm weight) and bf16 activations: the GEMM
  operands are bf16 and every sum is exact here, rounded to fp32;
* "the input of the up-projections" is h = RMSNorm(x) (bf16), which also
  feeds the router; its FP8 copy (hq, hs) is what the backward reads for
  every weight gradient that needs h (gate, up and router);
* "the input of SwiGLU" is the pair (g, u) of gate and up outputs (fp32
  sums); their FP8 copies, 1x128 along the hidden dimension of each row, are
  what the backward recomputes a = silu(g) u and the SwiGLU derivatives from;
* intermediates between the backward GEMMs are bf16 operands of the next
  BF16 GEMM: a (recomputed), w * dy (the routed weight times the output
  gradient), dg and du, and the dequantised h;
* the routing selection (top-k on the biased scores) passes no gradient;
  the weights w = c s_e / sum_j s_j (renormalised) or c s_e pass theirs to
  the sigmoid scores s = sigmoid(z), z = h W_r^T; the correction bias gets
  none;
* the bf16 rounding of h is passed straight through (derivative 1);
* outputs: dx (fp32), the norm weight's gradient (fp32), the router
  weight's gradient (fp32) and every expert's dW_gate, dW_up, dW_down (fp32,
  nn.Linear layout), all as sums over the whole batch.

``exact=True`` switches off every storage compression and bf16 rounding of
an intermediate (fp32 roundings of sums stay): the plain gradient of the
forward, which tests/test_oracle_train.py pins to torch autograd.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .fp8 import E4M3_MAX, bf16_round, e4m3_decode, e4m3_encode, f32
from .moe_ref import (LayerParams, dequantize_1x128, permute, quantize_1x128, rmsnorm, route,
                      silu_mul)


@dataclass
class TrainWeights:
    """bf16 values held in float32 arrays; G = routed + shared experts."""
    gate: np.ndarray      # [G, I, d]
    up: np.ndarray        # [G, I, d]
    down: np.ndarray      # [G, d, I]
    w_router: np.ndarray  # [E, d]


def _silu(g):
    return g / (1.0 + np.exp(-g))


def _dsilu(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def _rows_of(p: LayerParams, ids: np.ndarray):
    """(token, weight slot, expert) of every row: routed pairs in expert
    order (the permutation), then one shared row per token and shared expert."""
    T, k = ids.shape
    offsets, row_pair, _ = permute(ids, p.n_experts)
    tok = list(row_pair // k)
    slot = list(row_pair % k)
    grp = list(np.repeat(np.arange(p.n_experts), np.diff(offsets)))
    for j in range(p.n_shared):
        tok += list(range(T))
        slot += [-1] * T
        grp += [p.n_experts + j] * T
    return np.array(tok, np.int64), np.array(slot, np.int64), np.array(grp, np.int64)


# ------------------------------------------------------------------ forward
def train_forward(p: LayerParams, x, norm_w, bias, W: TrainWeights, exact: bool = False,
                  experts=None) -> dict:
    """Forward of the training step on every token.  Returns the output, the
    routing, and what is stored for the backward: hq/hs (FP8 copy of h) and,
    per row in permuted order, the FP8 copies of g and u.  ``experts``
    restricts the expert rows computed to those groups (the routing still
    covers every token; y and out are then partial)."""
    T = x.shape[0]
    h = rmsnorm(x, norm_w, p.rms_eps, round_bf16=True)
    hq, hs = quantize_1x128(h)
    r = route(h, W.w_router, bias, p.top_k, p.routed_scaling, p.norm_topk_prob)
    ids, w, s = r["ids"], r["w"], r["s"]
    ssel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    tok, slot, grp = _rows_of(p, ids)
    R, I = len(tok), p.d_ff
    g = np.zeros((R, I), np.float32)
    u = np.zeros((R, I), np.float32)
    o = np.zeros((R, p.d_model), np.float32)
    gq, uq = np.zeros((R, I), np.uint8), np.zeros((R, I), np.uint8)
    gsc, usc = np.ones((R, I // 128), np.float32), np.ones((R, I // 128), np.float32)
    gfrag, ufrag = np.zeros((R, I), bool), np.zeros((R, I), bool)
    for e in (np.unique(grp) if experts is None else experts):
        rr = np.nonzero(grp == e)[0]
        if len(rr) == 0:
            continue
        hin = h[tok[rr]].astype(np.float64)
        g[rr] = f32(hin @ W.gate[e].astype(np.float64).T)
        u[rr] = f32(hin @ W.up[e].astype(np.float64).T)
        gq[rr], gsc[rr] = quantize_1x128(g[rr])
        uq[rr], usc[rr] = quantize_1x128(u[rr])
        ah = np.abs(hin)
        gfrag[rr] = fragile_1x128(g[rr], gsc[rr], ah @ np.abs(W.gate[e].astype(np.float64)).T)
        ufrag[rr] = fragile_1x128(u[rr], usc[rr], ah @ np.abs(W.up[e].astype(np.float64)).T)
        a = silu_mul(g[rr], u[rr])
        a = a if exact else bf16_round(a)
        o[rr] = f32(a.astype(np.float64) @ W.down[e].astype(np.float64).T)
    # y: the token's routed rows in ascending expert id times their weight,
    # then the shared rows; out = x + y rounded once to bf16
    wr = np.where(slot >= 0, w[tok, np.maximum(slot, 0)], 1.0).astype(np.float64)
    y64 = np.zeros((T, p.d_model))
    np.add.at(y64, tok, wr[:, None] * o.astype(np.float64))
    y = f32(y64)
    out = bf16_round(f32(f32(x) + y))
    return dict(h=h, hq=hq, hs=hs, ids=ids, w=w, s=ssel, tok=tok, slot=slot, grp=grp,
                g=g, u=u, gq=gq, gs=gsc, uq=uq, us=usc, gfrag=gfrag, ufrag=ufrag, o=o, y=y,
                out=out)


def forward_rows(fwd: dict, W: TrainWeights, e: int, rows) -> None:
    """Fill in the forward's g, u, their kept copies and fragility for some
    rows of group e (in place; for checking a subset of a large group)."""
    rows = np.asarray(rows, np.int64)
    hin = fwd["h"][fwd["tok"][rows]].astype(np.float64)
    ah = np.abs(hin)
    for name, mat, q, sc, fr in (("g", W.gate[e], "gq", "gs", "gfrag"),
                                 ("u", W.up[e], "uq", "us", "ufrag")):
        m = mat.astype(np.float64)
        v = f32(hin @ m.T)
        fwd[name][rows] = v
        fwd[q][rows], fwd[sc][rows] = quantize_1x128(v)
        fwd[fr][rows] = fragile_1x128(v, fwd[sc][rows], ah @ np.abs(m).T)


# ----------------------------------------------------------------- backward
def stored_inputs(fwd: dict, rows, exact: bool = False):
    """What the backward reads for rows: h of their tokens (dequantised FP8
    copy, as bf16 operand) and g, u (dequantised FP8 copies, fp32)."""
    rows = np.asarray(rows, np.int64)
    tok = fwd["tok"][rows]
    if exact:
        return (fwd["h"][tok].astype(np.float64), fwd["g"][rows].astype(np.float64),
                fwd["u"][rows].astype(np.float64))
    ht = bf16_round(f32(dequantize_1x128(fwd["hq"][tok], fwd["hs"][tok]))).astype(np.float64)
    gt = f32(dequantize_1x128(fwd["gq"][rows], fwd["gs"][rows])).astype(np.float64)
    ut = f32(dequantize_1x128(fwd["uq"][rows], fwd["us"][rows])).astype(np.float64)
    return ht, gt, ut


# Window around a rounding midpoint within which a value counts as fragile:
# 2^-14 of the value, plus 2^-20 of the sum of the absolute terms of the dot
# product behind it (an fp32 sum formed in another order, as the GPU forms
# it, differs from the exact one by far less than that; where the terms
# cancel, that absolute part is what matters).  Elsewhere both sides round
# to the same bf16 value or e4m3 code.
FRAGILE_REL = 2.0 ** -14
ACC_REL = 2.0 ** -20


def fragile_bf16(v, abs_sum=0.0) -> np.ndarray:
    """Where the fp32 value v lies so close to the midpoint between two bf16
    neighbours that a slightly different fp32 sum may round the other way."""
    v64 = f32(v).astype(np.float64)
    win = FRAGILE_REL * np.abs(v64) + ACC_REL * np.asarray(abs_sum, np.float64)
    return bf16_round(f32(v64 + win)) != bf16_round(f32(v64 - win))


def fragile_1x128(a, scales, abs_sum=0.0) -> np.ndarray:
    """Where an fp32 value's quotient by its 1x128 scale lies so close to the
    midpoint between two e4m3 codes that a slightly different fp32 value
    (another summation order) may take the other code."""
    a = f32(a).astype(np.float64)
    sc = np.repeat(scales.astype(np.float64), 128, axis=1)
    q = a / sc
    win = FRAGILE_REL * np.abs(q) + ACC_REL * np.asarray(abs_sum, np.float64) / sc
    up = e4m3_encode(np.clip(f32(q + win), -E4M3_MAX, E4M3_MAX))
    dn = e4m3_encode(np.clip(f32(q - win), -E4M3_MAX, E4M3_MAX))
    return up != dn


def e4m3_step(codes, scales) -> np.ndarray:
    """Value distance to the farther e4m3 neighbour of each code, scaled:
    2^(floor(log2|v|) - 3) for normal values, 2^-9 below 2^-6."""
    v = np.abs(e4m3_decode(codes))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.exp2(e - 3) * np.repeat(scales.astype(np.float64), 128, axis=1)


def _d2silu(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 - s) * (2.0 + g * (1.0 - 2.0 * s))


def expert_backward(p: LayerParams, fwd: dict, dout, W: TrainWeights, e: int, rows,
                    exact: bool = False) -> dict:
    """Backward through expert e for some of its rows (all of them for its
    weight gradients).  dy of a row is dout of its token (the residual passes
    dout unchanged to x, and y enters out with weight 1).

      da_raw = W_down^T dy                   (fp32)
      dw     = a~ . da_raw                    (routed rows: the weight's gradient)
      da     = w da_raw ;  dg = da u~ silu'(g~) ;  du = da silu(g~)
      dh_row = W_gate^T dg + W_up^T du        (fp32)
      dW_down = sum_rows (w dy) a~^T ; dW_gate = sum dg h~^T ; dW_up = sum du h~^T
    with a~ = silu(g~) u~ from the stored copies."""
    rows = np.asarray(rows, np.int64)
    tok, slot = fwd["tok"][rows], fwd["slot"][rows]
    routed = slot >= 0
    wr = np.where(routed, fwd["w"][tok, np.maximum(slot, 0)], np.float32(1.0)).astype(np.float64)
    ht, gt, ut = stored_inputs(fwd, rows, exact)
    dy = f32(dout[tok]).astype(np.float64)
    wg, wu, wd = (W.gate[e].astype(np.float64), W.up[e].astype(np.float64),
                  W.down[e].astype(np.float64))
    at = f32(_silu(gt) * ut).astype(np.float64)
    da_raw = f32(dy @ wd).astype(np.float64)
    dw = f32(np.sum(at * da_raw, axis=1))
    da = wr[:, None] * da_raw
    dg = da * ut * _dsilu(gt)
    du = da * _silu(gt)
    dg_pre, du_pre = dg, du
    if not exact:
        dg, du = bf16_round(f32(dg)).astype(np.float64), bf16_round(f32(du)).astype(np.float64)
    dh_row = f32(dg @ wg + du @ wu)
    dyw = wr[:, None] * dy
    a_op = at
    # Error model (what another valid evaluation may differ by, elementwise):
    # (1) a bf16 operand whose fp32 value is fragile may be the other
    #     neighbour, one bf16 step (<= 2^-7 of it) away;
    # (2) a kept g or u code that is fragile (fwd["gfrag"], fwd["ufrag"]) may
    #     be the neighbouring e4m3 code, one e4m3 step away; the steps move
    #     a~, dg and du by at most their first-order sensitivities times the
    #     step (x1.5 for the curvature over one step and the bf16 rounding of
    #     the moved value).
    # The bounds are sums of those moves over each output's terms.
    fr = {}
    if not exact:
        s_da = np.abs(wr)[:, None] * (np.abs(dy) @ np.abs(wd))   # terms of w da_raw
        fr["dg"] = fragile_bf16(dg_pre, s_da * np.abs(ut * _dsilu(gt)))
        fr["du"] = fragile_bf16(du_pre, s_da * np.abs(_silu(gt)))
        fr["dyw"], fr["a"] = fragile_bf16(dyw), fragile_bf16(at)
        dyw = bf16_round(f32(dyw)).astype(np.float64)
        a_op = bf16_round(f32(at)).astype(np.float64)
    bounds = {}
    if fr:
        step = 2.0 ** -7
        ddg = step * np.abs(dg) * fr["dg"]
        ddu = step * np.abs(du) * fr["du"]
        dda = step * np.abs(a_op) * fr["a"]
        ddyw = step * np.abs(dyw) * fr["dyw"]
        if "gfrag" in fwd:
            dgs = fwd["gfrag"][rows] * e4m3_step(fwd["gq"][rows], fwd["gs"][rows])
            dus = fwd["ufrag"][rows] * e4m3_step(fwd["uq"][rows], fwd["us"][rows])
            k = 1.5
            dda = dda + k * (np.abs(_dsilu(gt) * ut) * dgs + np.abs(_silu(gt)) * dus)
            ddg = ddg + k * np.abs(da) * (np.abs(ut * _d2silu(gt)) * dgs + np.abs(_dsilu(gt)) * dus)
            ddu = ddu + k * np.abs(da * _dsilu(gt)) * dgs
        aht = np.abs(ht)
        bounds = dict(
            bound_gate=ddg.T @ aht, bound_up=ddu.T @ aht,
            bound_down=ddyw.T @ np.abs(a_op) + np.abs(dyw).T @ dda,
            bound_dh_row=ddg @ np.abs(wg) + ddu @ np.abs(wu),
            bound_dw=np.where(routed, np.sum(np.abs(da_raw) * dda, axis=1), 0.0))
    return dict(rows=rows, da_raw=f32(da_raw), dw=np.where(routed, dw, np.float32(0.0)),
                dg=f32(dg), du=f32(du), dh_row=dh_row,
                dW_down=f32(dyw.T @ a_op), dW_gate=f32(dg.T @ ht), dW_up=f32(du.T @ ht),
                **bounds)


def router_norm_backward(p: LayerParams, fwd: dict, x, norm_w, W: TrainWeights, dout, dh,
                         dw, exact: bool = False, tokens=None, bounds=None) -> dict:
    """Backward through the routing weights, the router and RMSNorm.

    dw [T, k]: gradient of each routed weight; dh [T, d]: gradient of h from
    the experts.  Renormalised weights w_j = c s_j / S, S = sum_i s_i:
      ds_j = c (dw_j / S - sum_i dw_i s_i / S^2)     (c ds_j without renorm)
      dz_j = ds_j s_j (1 - s_j)
      dh  += sum_j dz_j W_r[id_j] ;  dW_r[id_j] += dz_j h~
    RMSNorm, h = gamma x r, r = (mean(x^2) + eps)^-1/2:
      dx = dout + r (gamma dh) - x r^3 / d * sum(gamma dh x) ;  dgamma = sum_t dh x r
    ``tokens`` restricts dx to those tokens (dW_r and dgamma need all)."""
    T, k = fwd["ids"].shape
    ids = fwd["ids"].astype(np.int64)
    s = fwd["s"].astype(np.float64)
    c = float(np.float32(p.routed_scaling))
    dw64 = dw.astype(np.float64)
    if p.norm_topk_prob:
        S = s.sum(axis=1, keepdims=True)
        ds = c * (dw64 / S - np.sum(dw64 * s, axis=1, keepdims=True) / S ** 2)
    else:
        ds = c * dw64
    dz = ds * s * (1.0 - s)
    wr = W.w_router.astype(np.float64)
    dh_tot = dh.astype(np.float64) + np.einsum("tj,tjd->td", dz, wr[ids])
    ht = (fwd["h"].astype(np.float64) if exact else
          bf16_round(f32(dequantize_1x128(fwd["hq"], fwd["hs"]))).astype(np.float64))
    dWr = np.zeros((p.n_experts, p.d_model))
    np.add.at(dWr, ids.reshape(-1), (dz.reshape(-1)[:, None] * np.repeat(ht, k, axis=0)))
    x64 = f32(x).astype(np.float64)
    d = x64.shape[1]
    ms = np.mean(x64 ** 2, axis=1, keepdims=True)
    r = 1.0 / np.sqrt(ms + p.rms_eps)
    gam = f32(norm_w).astype(np.float64)[None, :]
    gdh = gam * dh_tot
    dx = (f32(dout).astype(np.float64) + r * gdh
          - x64 * r ** 3 / d * np.sum(gdh * x64, axis=1, keepdims=True))
    dgamma = np.sum(dh_tot * x64 * r, axis=0)
    sel = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    out = dict(dz=f32(dz), dh_total=f32(dh_tot), dx=f32(dx[sel]), d_norm_w=f32(dgamma),
               d_w_router=f32(dWr), tokens=sel)
    if bounds is not None:
        # the error model carried through: bounds (nonnegative) on dh [T, d]
        # and dw [T, k] move ds, dz, dh_total, dx, dgamma and dW_r by at most
        # the absolute values of the same linear maps applied to them
        bdh, bdw = bounds
        if p.norm_topk_prob:
            bds = c * (bdw / S + np.sum(bdw * s, axis=1, keepdims=True) / S ** 2)
        else:
            bds = c * bdw
        bdz = bds * s * (1.0 - s)
        bdh_tot = bdh + np.einsum("tj,tjd->td", bdz, np.abs(wr[ids]))
        agam = np.abs(gam)
        bdx = (r * agam * bdh_tot
               + np.abs(x64) * r ** 3 / d * np.sum(agam * np.abs(x64) * bdh_tot, axis=1,
                                                   keepdims=True))
        bWr = np.zeros((p.n_experts, p.d_model))
        np.add.at(bWr, ids.reshape(-1), bdz.reshape(-1)[:, None] * np.repeat(np.abs(ht), k, axis=0))
        out.update(bound_dx=bdx[sel], bound_d_norm_w=np.sum(bdh_tot * np.abs(x64) * r, axis=0),
                   bound_d_w_router=bWr)
    return out


def train_backward(p: LayerParams, fwd: dict, x, norm_w, W: TrainWeights, dout,
                   exact: bool = False) -> dict:
    """The whole backward on every token and expert (small layers)."""
    T, k = fwd["ids"].shape
    R = len(fwd["tok"])
    dh_rows = np.zeros((R, p.d_model), np.float32)
    dw_rows = np.zeros(R, np.float32)
    G = p.n_experts + p.n_shared
    dW = {"gate": np.zeros((G, p.d_ff, p.d_model), np.float32),
          "up": np.zeros((G, p.d_ff, p.d_model), np.float32),
          "down": np.zeros((G, p.d_model, p.d_ff), np.float32)}
    bound = {n: np.zeros(dW[n].shape) for n in dW} if not exact else None
    b_rows = np.zeros((R, p.d_model)) if bound is not None else None
    b_dw_rows = np.zeros(R) if bound is not None else None
    for e in range(G):
        rows = np.nonzero(fwd["grp"] == e)[0]
        if len(rows) == 0:
            continue
        b = expert_backward(p, fwd, dout, W, e, rows, exact)
        dh_rows[rows] = b["dh_row"]
        dw_rows[rows] = b["dw"]
        dW["gate"][e], dW["up"][e], dW["down"][e] = b["dW_gate"], b["dW_up"], b["dW_down"]
        if bound is not None:
            bound["gate"][e], bound["up"][e], bound["down"][e] = (b["bound_gate"], b["bound_up"],
                                                                  b["bound_down"])
            b_rows[rows] = b["bound_dh_row"]
            b_dw_rows[rows] = b["bound_dw"]
    # dh of a token: its routed rows in ascending expert id, then its shared rows
    dh64 = np.zeros((T, p.d_model))
    np.add.at(dh64, fwd["tok"], dh_rows.astype(np.float64))
    dh = f32(dh64)
    dw = np.zeros((T, k), np.float32)
    routed = fwd["slot"] >= 0
    dw[fwd["tok"][routed], fwd["slot"][routed]] = dw_rows[routed]
    bnd = None
    if bound is not None:
        bdh = np.zeros((T, p.d_model))
        np.add.at(bdh, fwd["tok"], b_rows)
        bdw = np.zeros((T, k))
        bdw[fwd["tok"][routed], fwd["slot"][routed]] = b_dw_rows[routed]
        bnd = (bdh, bdw)
    rn = router_norm_backward(p, fwd, x, norm_w, W, dout, dh, dw, exact, bounds=bnd)
    extra = {} if bound is None else dict(bound_dh_rows=b_rows, bound_dw=bdw)
    return dict(dh_rows=dh_rows, dw=dw, dh=dh, dW=dW, dW_bound=bound, **extra, **rn)
