"""Pins of the training-step oracle (oracle/train_ref.py), CPU only.

1. Exact mode against torch autograd (float64): every gradient the oracle
   forms by hand (dx, the norm weight's, the router weight's, each expert's
   dW_gate, dW_up, dW_down, the routing weights') equals the one torch
   derives from the same forward.
2. FP8 storage against torch with the same storage: custom autograd
   functions keep FP8 copies (the oracle's pinned 1x128 quantiser) of h and
   of (g, u), and recompute the forward from the copies in their backward,
   letting autograd form the derivatives.  The oracle's FP8 mode matches it
   to the bf16 rounding of its backward intermediates, and the exact
   gradient does not (so the pin sees which copies are read where).
3. A mutation pass: plausible mistakes planted in the oracle fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from oracle import train_ref as TR
from oracle.fp8 import bf16_round, f32


def _problem(seed=0, T=12, d=256, E=8, S=1, k=3, I=256, renorm=True):
    rng = np.random.default_rng(seed)
    p = R.LayerParams(d_model=d, n_experts=E, n_shared=S, top_k=k, d_ff=I, fp8=True,
                      norm_topk_prob=renorm)
    G = E + S
    b = lambda a: bf16_round(f32(a))
    x = b(rng.standard_normal((T, d)))
    norm_w = b(1.0 + 0.1 * rng.standard_normal(d))
    bias = f32(0.01 * rng.standard_normal(E))
    W = TR.TrainWeights(gate=b(0.05 * rng.standard_normal((G, I, d))),
                        up=b(0.05 * rng.standard_normal((G, I, d))),
                        down=b(0.05 * rng.standard_normal((G, d, I))),
                        w_router=b(0.1 * rng.standard_normal((E, d))))
    dout = b(rng.standard_normal((T, d)))
    return p, x, norm_w, bias, W, dout


def _q(a):
    """FP8 1x128 copy of a float64 tensor, dequantised (the oracle's quantiser)."""
    codes, scales = R.quantize_1x128(f32(a.detach().numpy()))
    return torch.from_numpy(R.dequantize_1x128(codes, scales))


class _StoredLinear(torch.autograd.Function):
    """y = x W^T; the weight gradient reads an FP8 copy of x, bf16-rounded."""

    @staticmethod
    def forward(ctx, x, w):
        ctx.save_for_backward(torch.from_numpy(bf16_round(f32(_q(x).numpy()))).double(), w)
        return x @ w.T

    @staticmethod
    def backward(ctx, gy):
        xs, w = ctx.saved_tensors
        return gy @ w, gy.T @ xs


class _StoredSwiGLUDown(torch.autograd.Function):
    """w * W_down (silu(g) u) for rows with routing weight w; the backward
    recomputes it from FP8 copies of g, u (nothing else of the expert is
    kept), so the routing weight's gradient also sees the recomputed output."""

    @staticmethod
    def forward(ctx, g, u, wd, wt):
        ctx.save_for_backward(_q(g), _q(u), wd, wt)
        return wt[:, None] * ((torch.nn.functional.silu(g) * u) @ wd.T)

    @staticmethod
    def backward(ctx, go):
        gs, us, wd, wt = ctx.saved_tensors
        with torch.enable_grad():
            g = gs.clone().requires_grad_(True)
            u = us.clone().requires_grad_(True)
            w = wd.detach().clone().requires_grad_(True)
            r = wt.detach().clone().requires_grad_(True)
            o = r[:, None] * ((torch.nn.functional.silu(g) * u) @ w.T)
            return torch.autograd.grad(o, (g, u, w, r), go)


def _torch_step(p, x, norm_w, W, dout, fwd, stored):
    """The forward in float64 torch with the oracle's routing choice and bf16
    h values (passed straight through), then autograd of sum(out * dout)."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    X, G_, WR = t(x), t(norm_w), t(W.w_router)
    WG, WU, WD = t(W.gate), t(W.up), t(W.down)
    ms = (X ** 2).mean(dim=1, keepdim=True)
    h = X / torch.sqrt(ms + p.rms_eps) * G_
    h = h + (torch.from_numpy(fwd["h"].astype(np.float64)) - h).detach()
    lin = _StoredLinear.apply if stored else (lambda a, w: a @ w.T)
    z = lin(h, WR)
    s = torch.sigmoid(z)
    ids = torch.from_numpy(fwd["ids"].astype(np.int64))
    sel = s.gather(1, ids)
    c = float(np.float32(p.routed_scaling))
    w = c * sel / sel.sum(dim=1, keepdim=True) if p.norm_topk_prob else c * sel
    y = torch.zeros_like(X)
    tok, slot, grp = fwd["tok"], fwd["slot"], fwd["grp"]
    for e in np.unique(grp):
        rr = np.nonzero(grp == e)[0]
        hin = h[torch.from_numpy(tok[rr])]
        g, u = lin(hin, WG[e]), lin(hin, WU[e])
        sl = slot[rr]
        wt = torch.where(torch.from_numpy(sl >= 0),
                         w[torch.from_numpy(tok[rr]), torch.from_numpy(np.maximum(sl, 0))],
                         torch.ones(len(rr), dtype=torch.float64))
        o = (_StoredSwiGLUDown.apply(g, u, WD[e], wt) if stored else
             wt[:, None] * ((torch.nn.functional.silu(g) * u) @ WD[e].T))
        y = y.index_add(0, torch.from_numpy(tok[rr]), o)
    out = X + y
    (out * torch.from_numpy(dout.astype(np.float64))).sum().backward()
    return dict(y=y.detach().numpy(), dx=X.grad.numpy(), d_norm_w=G_.grad.numpy(),
                d_w_router=WR.grad.numpy(), gate=WG.grad.numpy(), up=WU.grad.numpy(),
                down=WD.grad.numpy())


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def _compare(ob, ref, tol):
    errs = {"dx": _rel(ob["dx"], ref["dx"]), "d_norm_w": _rel(ob["d_norm_w"], ref["d_norm_w"]),
            "d_w_router": _rel(ob["d_w_router"], ref["d_w_router"])}
    for m in ("gate", "up", "down"):
        errs[m] = _rel(ob["dW"][m], ref[m])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return errs


@pytest.mark.parametrize("seed,renorm", [(0, True), (1, True), (2, False)])
def test_exact_gradient_matches_torch_autograd(seed, renorm):
    p, x, norm_w, bias, W, dout = _problem(seed, renorm=renorm)
    fwd = TR.train_forward(p, x, norm_w, bias, W, exact=True)
    ob = TR.train_backward(p, fwd, x, norm_w, W, dout, exact=True)
    ref = _torch_step(p, x, norm_w, W, dout, fwd, stored=False)
    assert _rel(fwd["y"], ref["y"]) < 1e-6        # the forward itself
    _compare(ob, ref, 1e-5)


def test_fp8_storage_matches_torch_with_the_same_storage():
    p, x, norm_w, bias, W, dout = _problem(4)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    ob = TR.train_backward(p, fwd, x, norm_w, W, dout)
    ref = _torch_step(p, x, norm_w, W, dout, fwd, stored=True)
    # the remaining difference is the bf16 rounding of the oracle's backward
    # intermediates (<= 4e-3 of the largest value on these problems)
    errs = _compare(ob, ref, 8e-3)
    # the exact gradient is several times further from the stored-copy
    # gradient on every output: the copies change the result
    ex = TR.train_backward(p, TR.train_forward(p, x, norm_w, bias, W, exact=True), x, norm_w, W,
                           dout, exact=True)
    far = _compare(ex, ref, 1.0)
    assert all(far[k] > 3 * errs[k] for k in errs), (far, errs)


def test_fp8_copies_are_the_pinned_quantiser_output():
    p, x, norm_w, bias, W, _ = _problem(5)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    hq, hs = R.quantize_1x128(fwd["h"])
    assert np.array_equal(hq, fwd["hq"]) and np.array_equal(hs, fwd["hs"])
    gq, gs = R.quantize_1x128(fwd["g"])
    assert np.array_equal(gq, fwd["gq"]) and np.array_equal(gs, fwd["gs"])
    # stored values are within one e4m3 step of the fp32 ones
    gt = R.dequantize_1x128(fwd["gq"], fwd["gs"])
    step = np.maximum(np.abs(fwd["g"]) * 2.0 ** -3,
                      np.repeat(fwd["gs"], 128, axis=1) * 2.0 ** -9)
    assert np.all(np.abs(gt - fwd["g"]) <= step)


def test_zero_output_gradient_gives_zero_gradients():
    p, x, norm_w, bias, W, dout = _problem(6)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    ob = TR.train_backward(p, fwd, x, norm_w, W, dout * 0)
    assert not np.any(ob["dx"]) and not np.any(ob["d_w_router"])
    assert not any(np.any(v) for v in ob["dW"].values())


def test_unused_expert_has_zero_weight_gradient():
    p, x, norm_w, bias, W, dout = _problem(7, T=2, E=16, k=2)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    ob = TR.train_backward(p, fwd, x, norm_w, W, dout)
    unused = sorted(set(range(p.n_experts)) - set(fwd["ids"].reshape(-1).tolist()))
    assert unused
    for e in unused:
        assert not np.any(ob["dW"]["gate"][e]) and not np.any(ob["d_w_router"][e])


# ------------------------------------------------------------ mutation pass
def _plant(mp, name, fn):
    mp.setattr(TR, name, fn)


MUTATIONS = {
    "silu derivative without its second term": ("_dsilu", lambda g: 1.0 / (1.0 + np.exp(-g))),
    "silu derivative of a sigmoid gate": ("_dsilu",
                                          lambda g: np.exp(-g) / (1.0 + np.exp(-g)) ** 2),
}


def _wrap_router(mp, post):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return post(orig(p, fwd, x, norm_w, W, dout, dh, dw, exact, tokens, bounds))
    mp.setattr(TR, "router_norm_backward", f)


def _wrap_expert(mp, pre=None, post=None):
    orig = TR.expert_backward

    def f(p, fwd, dout, W, e, rows, exact=False):
        if pre:
            fwd = pre(fwd)
        return post(orig(p, fwd, dout, W, e, rows, exact)) if post else orig(p, fwd, dout, W, e, rows, exact)
    mp.setattr(TR, "expert_backward", f)


def _no_routed_weight(mp):
    orig = TR.expert_backward

    def f(p, fwd, dout, W, e, rows, exact=False):
        f2 = dict(fwd)
        f2["w"] = np.ones_like(fwd["w"])
        return orig(p, f2, dout, W, e, rows, exact)
    mp.setattr(TR, "expert_backward", f)


def _renorm_sign(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return orig(p, fwd, x, norm_w, W, dout, dh, -dw, exact, tokens, bounds)
    mp.setattr(TR, "router_norm_backward", f)


def _no_residual_grad(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        r = orig(p, fwd, x, norm_w, W, dout, dh, dw, exact, tokens, bounds)
        r["dx"] = f32(r["dx"] - f32(dout))
        return r
    mp.setattr(TR, "router_norm_backward", f)


def _stored_not_used(mp):
    orig = TR.stored_inputs
    mp.setattr(TR, "stored_inputs", lambda fwd, rows, exact=False: orig(fwd, rows, True))


def _down_grad_transposed(mp):
    _wrap_expert(mp, post=lambda b: {**b, "dW_down": (b["dW_down"].reshape(-1)[::-1]
                                                      .reshape(b["dW_down"].shape))})


def _no_norm_weight(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return orig(p, fwd, x, np.ones_like(norm_w), W, dout, dh, dw, exact, tokens, bounds)
    mp.setattr(TR, "router_norm_backward", f)


FN_MUTATIONS = {
    "routed weight left out of da": _no_routed_weight,
    "renormalisation gradient with the wrong sign": _renorm_sign,
    "residual gradient dropped": _no_residual_grad,
    "fp32 g, u, h read instead of the stored copies": _stored_not_used,
    "dW_down laid out wrongly": _down_grad_transposed,
    "norm weight left out of the RMSNorm backward": _no_norm_weight,
}

PINS = [lambda: test_exact_gradient_matches_torch_autograd(0, True),
        lambda: test_exact_gradient_matches_torch_autograd(2, False),
        test_fp8_storage_matches_torch_with_the_same_storage]


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(FN_MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    if name in MUTATIONS:
        attr, fn = MUTATIONS[name]
        _plant(monkeypatch, attr, fn)
    else:
        FN_MUTATIONS[name](monkeypatch)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {name}"


def test_error_model_covers_an_fp32_level_change():
    """Another evaluation of the same step whose fp32 sums differ at the
    level of their rounding (here: the gate and down weights scaled by
    1 + 1e-7 noise, which moves g, da_raw, dg, du, a~ and w dy by about 1e-7
    relative) rounds some fragile bf16 operands and fragile kept e4m3 codes
    the other way; every output then stays within the bound the oracle
    states for it (one bf16 step of each fragile operand, one e4m3 step of
    each fragile code, carried through the backward)."""
    p, x, norm_w, bias, W, dout = _problem(11, T=200, d=256, E=16, k=4, I=256)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    ref = TR.train_backward(p, fwd, x, norm_w, W, dout)
    rng = np.random.default_rng(12)
    jig = lambda a: a.astype(np.float64) * (1.0 + 1e-7 * rng.standard_normal(a.shape))
    W2 = TR.TrainWeights(gate=jig(W.gate), up=W.up, w_router=W.w_router, down=jig(W.down))
    fwd2 = TR.train_forward(p, x, norm_w, bias, W2)
    assert np.array_equal(fwd2["ids"], fwd["ids"])
    flipped = (fwd2["gq"] != fwd["gq"]) | (fwd2["uq"] != fwd["uq"])
    assert flipped.any() and np.all(fwd["gfrag"][fwd2["gq"] != fwd["gq"]])
    alt = TR.train_backward(p, fwd2, x, norm_w, W2, dout)
    pairs = [(alt["dW"][n], ref["dW"][n], ref["dW_bound"][n]) for n in ("gate", "up", "down")]
    pairs += [(alt["dh_rows"], ref["dh_rows"], ref["bound_dh_rows"]),
              (alt["dw"], ref["dw"], ref["bound_dw"]), (alt["dx"], ref["dx"], ref["bound_dx"]),
              (alt["d_norm_w"], ref["d_norm_w"], ref["bound_d_norm_w"]),
              (alt["d_w_router"], ref["d_w_router"], ref["bound_d_w_router"])]
    worst = 0.0
    for a, r, bnd in pairs:
        diff = np.abs(a.astype(np.float64) - r)
        rms = np.sqrt(np.mean(r.astype(np.float64) ** 2))
        assert np.all(diff <= bnd + 1e-5 * rms)
        worst = max(worst, diff.max() / rms)
    assert worst > 1e-3      # the change is visible: fragile operands and codes did flip

# ------------------------------------------------------------ mutation pass
def _plant(mp, name, fn):
    mp.setattr(TR, name, fn)


MUTATIONS = {
    "silu derivative without its second term": ("_dsilu", lambda g: 1.0 / (1.0 + np.exp(-g))),
    "silu derivative of a sigmoid gate": ("_dsilu",
                                          lambda g: np.exp(-g) / (1.0 + np.exp(-g)) ** 2),
}


def _wrap_router(mp, post):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return post(orig(p, fwd, x, norm_w, W, dout, dh, dw, exact, tokens, bounds))
    mp.setattr(TR, "router_norm_backward", f)


def _wrap_expert(mp, pre=None, post=None):
    orig = TR.expert_backward

    def f(p, fwd, dout, W, e, rows, exact=False):
        if pre:
            fwd = pre(fwd)
        return post(orig(p, fwd, dout, W, e, rows, exact)) if post else orig(p, fwd, dout, W, e, rows, exact)
    mp.setattr(TR, "expert_backward", f)


def _no_routed_weight(mp):
    orig = TR.expert_backward

    def f(p, fwd, dout, W, e, rows, exact=False):
        f2 = dict(fwd)
        f2["w"] = np.ones_like(fwd["w"])
        return orig(p, f2, dout, W, e, rows, exact)
    mp.setattr(TR, "expert_backward", f)


def _renorm_sign(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return orig(p, fwd, x, norm_w, W, dout, dh, -dw, exact, tokens, bounds)
    mp.setattr(TR, "router_norm_backward", f)


def _no_residual_grad(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        r = orig(p, fwd, x, norm_w, W, dout, dh, dw, exact, tokens, bounds)
        r["dx"] = f32(r["dx"] - f32(dout))
        return r
    mp.setattr(TR, "router_norm_backward", f)


def _stored_not_used(mp):
    orig = TR.stored_inputs
    mp.setattr(TR, "stored_inputs", lambda fwd, rows, exact=False: orig(fwd, rows, True))


def _down_grad_transposed(mp):
    _wrap_expert(mp, post=lambda b: {**b, "dW_down": (b["dW_down"].reshape(-1)[::-1]
                                                      .reshape(b["dW_down"].shape))})


def _no_norm_weight(mp):
    orig = TR.router_norm_backward

    def f(p, fwd, x, norm_w, W, dout, dh, dw, exact=False, tokens=None, bounds=None):
        return orig(p, fwd, x, np.ones_like(norm_w), W, dout, dh, dw, exact, tokens, bounds)
    mp.setattr(TR, "router_norm_backward", f)


FN_MUTATIONS = {
    "routed weight left out of da": _no_routed_weight,
    "renormalisation gradient with the wrong sign": _renorm_sign,
    "residual gradient dropped": _no_residual_grad,
    "fp32 g, u, h read instead of the stored copies": _stored_not_used,
    "dW_down laid out wrongly": _down_grad_transposed,
    "norm weight left out of the RMSNorm backward": _no_norm_weight,
}

PINS = [lambda: test_exact_gradient_matches_torch_autograd(0, True),
        lambda: test_exact_gradient_matches_torch_autograd(2, False),
        test_fp8_storage_matches_torch_with_the_same_storage]


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(FN_MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    if name in MUTATIONS:
        attr, fn = MUTATIONS[name]
        _plant(monkeypatch, attr, fn)
    else:
        FN_MUTATIONS[name](monkeypatch)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {name}"


def test_error_model_covers_an_fp32_level_change():
    """Another evaluation of the same step whose fp32 sums differ at the
    level of their rounding (here: the down weights scaled by 1 + 1e-7 noise,
    which moves da_raw, dg, du, a~ and w dy by about 1e-7 relative) rounds
    some fragile bf16 operands the other way; every weight-gradient element
    then stays within the bound the oracle states for it (one bf16 step of
    each fragile operand in its sum).  At the Kimi K2 width one such step of
    a large operand moves an element by a few percent of the tensor's RMS."""
    p, x, norm_w, bias, W, dout = _problem(11, T=200, d=256, E=16, k=4, I=256)
    fwd = TR.train_forward(p, x, norm_w, bias, W)
    ref = TR.train_backward(p, fwd, x, norm_w, W, dout)
    rng = np.random.default_rng(12)
    W2 = TR.TrainWeights(gate=W.gate, up=W.up, w_router=W.w_router,
                         down=(W.down.astype(np.float64) *
                               (1.0 + 1e-7 * rng.standard_normal(W.down.shape))))
    alt = TR.train_backward(p, fwd, x, norm_w, W2, dout)
    worst_plain = 0.0
    for n in ("gate", "up", "down"):
        d = np.abs(alt["dW"][n].astype(np.float64) - ref["dW"][n])
        rms = np.sqrt(np.mean(ref["dW"][n].astype(np.float64) ** 2))
        assert np.all(d <= ref["dW_bound"][n] + 1e-5 * rms), n
        worst_plain = max(worst_plain, d.max() / rms)
    assert worst_plain > 1e-4      # the change is visible: fragile operands did flip
