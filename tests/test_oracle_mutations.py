"""The oracle's pins catch plausible mistakes: a mutation pass.

Each case plants one mistake in the CPU oracle (in this process only,
through monkeypatch) and then runs every pin of tests/test_oracle_pins.py and
tests/test_oracle_codec.py; at least one of them has to fail.  The mistakes
are the ones a from-the-pages implementation could plausibly make: the
biased score used as the expert weight, gate and up swapped, no
requantisation before the down projection, a scaled shared expert, another
RMSNorm epsilon, the MI300 e4m3 maximum (240) instead of OCP's 448, ties to
the higher expert id, tokens out of order inside an expert, no
renormalisation, softmax scores, SiLU replaced by a sigmoid gate, the weight
block scales or the activation block scales mapped to the wrong blocks, no
residual, the router rows misaligned, the correction bias ignored, h left
unrounded, e4m3 rounding toward zero and the sign of the top-k gap.

The unmutated pins pass in their own modules; nothing here touches the GPU.
"""
import numpy as np
import pytest

import test_oracle_codec as PC
import test_oracle_pins as PP
from oracle import adapt as A
from oracle import fp8 as F
from oracle import moe_ref as R

_MODULES = (F, R, A, PP, PC)


def _plant(monkeypatch, name, new):
    """Replace `name` in every module that holds the oracle's object for it."""
    hit = False
    orig = getattr(R, name, None)
    if orig is None:
        orig = getattr(F, name)
    for m in _MODULES:
        if getattr(m, name, None) is orig:
            monkeypatch.setattr(m, name, new)
            hit = True
    assert hit, name
    return orig


def _pin_calls():
    calls = []
    for mod in (PP, PC):
        for name in sorted(dir(mod)):
            fn = getattr(mod, name)
            if not (name.startswith("test_") and callable(fn)):
                continue
            marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            if not marks:
                calls.append((f"{mod.__name__}::{name}", fn, {}))
                continue
            assert len(marks) == 1, name
            argnames, values = marks[0].args[:2]
            names = ([a.strip() for a in argnames.split(",")] if isinstance(argnames, str)
                     else list(argnames))
            for v in values:
                v = getattr(v, "values", v)
                if len(names) == 1 and not (isinstance(v, tuple) and len(v) == 1):
                    v = (v,)
                calls.append((f"{mod.__name__}::{name}{list(v)}", fn, dict(zip(names, v))))
    return calls


# ---------------------------------------------------------------- mistakes ---
def _biased_weights(mp):
    route = R.route

    def mutated(h, w_router, bias, k, scaling, renorm):
        r = route(h, w_router, bias, k, scaling, renorm)
        r["w"] = R.routing_weights(r["sb"], r["ids"], scaling, renorm)
        return r
    _plant(mp, "route", mutated)


def _gate_up_swapped(mp):
    silu_mul = R.silu_mul
    _plant(mp, "silu_mul", lambda g, u: silu_mul(u, g))


def _no_requantisation(mp):
    swiglu = R.swiglu_expert

    def mutated(hrows, wg, wu, wd, fp8):
        o, a, c, s = swiglu(hrows, wg, wu, wd, fp8)
        if fp8:
            o = F.f32(a.astype(np.float64) @ wd.T)
        return o, a, c, s
    _plant(mp, "swiglu_expert", mutated)


def _rewrap_layer(mp, post):
    layer = R.moe_layer

    def mutated(p, x, *args, **kw):
        return post(p, x, layer(p, x, *args, **kw))
    _plant(mp, "moe_layer", mutated)


def _set_y(p, x, res, y):
    out = F.f32(F.f32(x[res["tokens"]]) + y)
    res["y"] = y
    res["out"] = F.bf16_round(out) if p.fp8 else out
    return res


def _shared_scaled(mp):
    def post(p, x, res):
        if not p.n_shared:
            return res
        y = F.f32(res["y"].astype(np.float64)
                  + (p.routed_scaling - 1.0) * res["shared"].astype(np.float64))
        return _set_y(p, x, res, y)
    _rewrap_layer(mp, post)


def _no_residual(mp):
    def post(p, x, res):
        res["out"] = F.bf16_round(res["y"]) if p.fp8 else res["y"].copy()
        return res
    _rewrap_layer(mp, post)


def _eps_1e5(mp):
    rmsnorm = R.rmsnorm

    def mutated(x, gamma, eps, round_bf16):
        return rmsnorm(x, gamma, 10.0 * eps, round_bf16)
    _plant(mp, "rmsnorm", mutated)


def _h_not_rounded(mp):
    rmsnorm = R.rmsnorm

    def mutated(x, gamma, eps, round_bf16):
        return rmsnorm(x, gamma, eps, False)
    _plant(mp, "rmsnorm", mutated)


def _e4m3_max_240(mp):
    mp.setattr(R, "E4M3_MAX", 240.0)


def _ties_to_higher_id(mp):
    def mutated(sb, k):
        T, E = sb.shape
        order = E - 1 - np.argsort(-sb[:, ::-1], axis=1, kind="stable")
        ids = np.sort(order[:, :k], axis=1).astype(np.int32)
        rows = np.arange(T)
        gap = (F.f32(sb[rows, order[:, k - 1]] - sb[rows, order[:, k]]) if k < E
               else np.full(T, np.inf, dtype=np.float32))
        return ids, gap
    _plant(mp, "select_topk", mutated)


def _gap_sign(mp):
    select = R.select_topk

    def mutated(sb, k):
        ids, gap = select(sb, k)
        return ids, np.where(np.isinf(gap), gap, -gap).astype(np.float32)
    _plant(mp, "select_topk", mutated)


def _tokens_descending_in_expert(mp):
    permute = R.permute

    def mutated(ids, n_experts):
        offsets, _, _ = permute(ids, n_experts)
        flat = ids.reshape(-1)
        row_pair = np.lexsort((-np.arange(flat.size), flat)).astype(np.int32)
        pair_row = np.empty_like(row_pair)
        pair_row[row_pair] = np.arange(flat.size, dtype=np.int32)
        return offsets, row_pair, pair_row
    _plant(mp, "permute", mutated)


def _no_renormalisation(mp):
    weights = R.routing_weights
    _plant(mp, "routing_weights", lambda s, ids, scaling, renorm: weights(s, ids, scaling, False))


def _softmax_scores(mp):
    def mutated(z):
        z64 = z.astype(np.float64)
        e = np.exp(z64 - z64.max(axis=-1, keepdims=True))
        return F.f32(e / e.sum(axis=-1, keepdims=True))
    _plant(mp, "sigmoid_scores", mutated)


def _sigmoid_gate(mp):
    def mutated(g, u):
        g64 = g.astype(np.float64)
        return F.f32(1.0 / (1.0 + np.exp(-g64)) * u.astype(np.float64))
    _plant(mp, "silu_mul", mutated)


def _weight_scales_misplaced(mp):
    dequant = R.dequantize_weight

    def mutated(codes, scales):
        return dequant(codes, np.ascontiguousarray(scales.T).reshape(scales.shape))
    _plant(mp, "dequantize_weight", mutated)


def _act_scales_reversed(mp):
    dequant = R.dequantize_1x128
    _plant(mp, "dequantize_1x128",
           lambda codes, scales: dequant(codes, np.ascontiguousarray(scales[:, ::-1])))


def _router_rows_shifted(mp):
    logits = R.router_logits
    _plant(mp, "router_logits", lambda h, w: logits(h, np.roll(w, 1, axis=0)))


def _bias_ignored(mp):
    route = R.route

    def mutated(h, w_router, bias, k, scaling, renorm):
        return route(h, w_router, np.zeros_like(bias), k, scaling, renorm)
    _plant(mp, "route", mutated)


def _e4m3_toward_zero(mp):
    encode = F.e4m3_encode

    def mutated(v):
        v = np.asarray(v, dtype=np.float32)
        codes = encode(v)
        over = np.abs(F.e4m3_decode(codes)) > np.abs(v.astype(np.float64))
        codes = codes.copy()
        codes[over] -= 1      # one step toward zero (magnitude bits are monotone)
        return codes
    _plant(mp, "e4m3_encode", mutated)


MUTATIONS = {
    "biased_weights": _biased_weights,
    "gate_up_swapped": _gate_up_swapped,
    "no_requantisation": _no_requantisation,
    "shared_scaled": _shared_scaled,
    "no_residual": _no_residual,
    "eps_1e-5": _eps_1e5,
    "h_not_rounded": _h_not_rounded,
    "e4m3_max_240": _e4m3_max_240,
    "ties_to_higher_id": _ties_to_higher_id,
    "gap_sign": _gap_sign,
    "tokens_descending_in_expert": _tokens_descending_in_expert,
    "no_renormalisation": _no_renormalisation,
    "softmax_scores": _softmax_scores,
    "sigmoid_gate": _sigmoid_gate,
    "weight_scales_misplaced": _weight_scales_misplaced,
    "act_scales_reversed": _act_scales_reversed,
    "router_rows_shifted": _router_rows_shifted,
    "bias_ignored": _bias_ignored,
    "e4m3_toward_zero": _e4m3_toward_zero,
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    caught, crashed = [], []
    for pin, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except AssertionError:
            caught.append(pin)
        except Exception as exc:        # not a catch: the planted code itself may be at fault
            crashed.append(f"{pin}: {type(exc).__name__}: {exc}")
    assert caught, f"no pin fails with the planted mistake {name!r} (crashes: {crashed})"


def test_unmutated_pins_pass_through_the_same_runner():
    """Control: the runner above calls every pin correctly, so a failure under
    a mutation is the mutation's doing."""
    calls = _pin_calls()
    assert len(calls) >= 30
    for pin, fn, kw in calls:
        fn(**kw)
