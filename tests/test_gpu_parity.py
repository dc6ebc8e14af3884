"""Parity of the HIP layer (through the C ABI) with the CPU oracle.

Small shapes are compared on every token; the Kimi K2 shapes (decode 64,
prefill 8192, skewed 16384, dense 4096 tokens) are run whole on the GPU in
the launch configuration the benchmark times, and compared on every token's
routing and permutation and on the outputs of sampled tokens, which the
oracle computes one expert at a time.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import moe_ref as R
from oracle.adapt import run_oracle, to_f32
from oracle.compare import MEAN_REL, assert_close, check_routing, close_report
from oracle.fp8 import bf16_round

pytestmark = pytest.mark.gpu

HAVE_GPU = torch.cuda.is_available()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not HAVE_GPU:
        pytest.skip("no GPU")
    from sparse_moe_transformer_sigmoid_amd import _lib
    _lib.load()          # raises if libk2moe.so is missing: no fallback path
    yield
    torch.cuda.synchronize()


def _log(msg):
    print(msg, flush=True)


def gpu_chain(layer, inp):
    """Unfused chain and fused forward on the GPU; numpy results."""
    x = inp.x
    T = x.shape[0]
    layer.use_router(inp)
    r = layer.router(x)
    pm = layer.permute(r.ids)
    rows, shared, act_q, act_s = layer.grouped_swiglu(T, r.xq, r.xs, pm.offsets, pm.row_pair,
                                                      return_act=True)
    y = layer.combine(rows, pm.pair_row, r.w, shared, residual=None, out_f32=True)
    out_u = layer.combine(rows, pm.pair_row, r.w, shared, residual=x)
    out_f = layer.forward(x)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return dict(ids=cpu(r.ids), w=cpu(r.w), gap=cpu(r.gap), xq=cpu(r.xq), xs=cpu(r.xs),
                offsets=cpu(pm.offsets), row_pair=cpu(pm.row_pair), pair_row=cpu(pm.pair_row),
                rows=rows, shared=shared, act_q=act_q, act_s=act_s,
                y=cpu(y), out_u=to_f32(out_u), out_f=to_f32(out_f))


def _gather(t, idx):
    return t[torch.from_numpy(np.asarray(idx).reshape(-1)).to(t.device).long()].cpu().numpy()


def check_requantised_codes(gpu_codes, gpu_scales, a_ref):
    """GPU SwiGLU codes against the oracle's exact quantisation of its own a.

    The codes are decided on fp32 values whose sums gfx950's FP8 MFMA forms at
    reduced precision (about 2^-16 of the sum of |products|).  A GPU code is
    accepted when its value is within one e4m3 step of the exact code's value,
    or within 1e-4 of the block maximum (values near zero, where cancellation
    makes the relative error large); at least 99% must be identical.
    """
    I = a_ref.shape[-1]
    codes, scales = R.quantize_1x128(a_ref.reshape(-1, I))
    gc = gpu_codes.reshape(codes.shape)
    gs = gpu_scales.reshape(scales.shape)
    same = float(np.mean(gc == codes))
    dq_g = R.dequantize_1x128(gc, scales)      # both codes in the oracle's scale;
    dq_r = R.dequantize_1x128(codes, scales)   # the scales are compared on their own
    amax = np.repeat(scales.astype(np.float64) * 448.0, 128, axis=1)
    step = np.abs(dq_r) * 2.0 ** -3
    excess = np.abs(dq_g - dq_r) - np.maximum(step, 1e-4 * amax)
    srel = float(np.max(np.abs(gs.astype(np.float64) / scales - 1.0)))
    _log(f"  swiglu codes: equal {same:.5f}, worst excess {excess.max():.2e}, "
         f"scale rel diff {srel:.2e}")
    assert same >= 0.99 and excess.max() <= 0 and srel <= 1e-3


def check_layer(inp, g, tokens=None, end_to_end=None):
    """Compare a gpu_chain result with the oracle on ``tokens`` (default all).

    Routing and the permutation are checked on every token.  Expert outputs
    of the compared tokens are evaluated by the oracle under the GPU's expert
    choice and, in the FP8 layer, on the GPU's requantised SwiGLU codes (each
    checked to be the exact code or one step from it); those are held to the
    output tolerance.  With end_to_end (default: d_ff >= 2048) the oracle's
    own exact path must also meet the output tolerance.
    """
    shape = inp.shape
    k, I = shape.top_k, shape.d_ff
    fp8 = shape.fmt == "fp8"
    T = inp.x.shape[0]
    P = T * k
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    if end_to_end is None:
        end_to_end = I >= 2048
    pidx = g["pair_row"].reshape(T, k)[sel]                        # [n, k] permuted rows
    ov = None
    if fp8:
        ov = dict(codes=_gather(g["act_q"], pidx).reshape(len(sel), k, I),
                  scales=_gather(g["act_s"], pidx).reshape(len(sel), k, -1))
        if shape.n_shared:
            ov["shared_codes"] = _gather(g["act_q"], P + sel)
            ov["shared_scales"] = _gather(g["act_s"], P + sel)
    ref = run_oracle(inp, tokens=sel, ids_override=g["ids"], act_override=ov)
    if not shape.dense:
        rep = check_routing(g["ids"], g["w"], ref)
        _log(f"  routing: {rep}")
    else:
        assert np.all(g["ids"] == 0) and np.all(g["w"] == np.float32(shape.routed_scaling))
    # permutation: bit-exact against the oracle's grouping of the GPU's ids
    off, rp, pr = R.permute(g["ids"], shape.n_experts)
    assert np.array_equal(g["offsets"], off)
    assert np.array_equal(g["row_pair"], rp)
    assert np.array_equal(g["pair_row"], pr)
    # fused forward is the unfused chain, bit for bit
    assert np.array_equal(g["out_f"].view(np.uint32), g["out_u"].view(np.uint32))
    rows = _gather(g["rows"], pidx).reshape(len(sel), k, -1)
    sh = _gather(g["shared"], sel) if shape.n_shared else None
    if fp8:
        assert np.array_equal(g["xs"][sel], ref["xs"]), "activation scales differ"
        xq_eq = np.mean(g["xq"][sel] == ref["xq"])
        assert xq_eq >= 0.9999, f"activation codes equal on {xq_eq:.6f}"
        check_requantised_codes(ov["codes"], ov["scales"], ref["a_pairs"])
        sfx = "_ov"
    else:
        assert_close(g["xq"][sel], ref["h"][sel], "h")
        sfx = ""
    rep_rows = assert_close(rows, ref["o_pairs" + sfx], "expert rows")
    if shape.n_shared:
        assert_close(sh, ref["shared" + sfx], "shared expert")
    rep_y = assert_close(g["y"][sel], ref["y" + sfx], "y (MoE output)")
    rep_o = assert_close(g["out_f"][sel], ref["out" + sfx], "out", bf16_out=fp8)
    _log(f"  rows {rep_rows}\n  y {rep_y}\n  out {rep_o}")
    if fp8:
        e2e_y = close_report(g["y"][sel], ref["y"])
        e2e_o = close_report(g["out_f"][sel], ref["out"], bf16_out=True)
        _log(f"  end to end vs exact oracle: y {e2e_y}\n  out {e2e_o}")
        assert e2e_y["mean_rel"] <= MEAN_REL and e2e_o["mean_rel"] <= MEAN_REL
        if end_to_end:
            assert e2e_y["ok"] and e2e_o["ok"], "end-to-end tolerance"
    return ref


def _layer(inp):
    from sparse_moe_transformer_sigmoid_amd.layer import K2MoE
    return K2MoE(inp)


# ------------------------------------------------------------- small shapes
def test_tiny_fp32_layer():
    inp = synth.generate(synth.TINY, seed=0, device="cuda")
    g = gpu_chain(_layer(inp), inp)
    check_layer(inp, g)


SMALL = [
    # (tokens, d_model, experts, shared, top_k, d_ff, seed) -- ragged token counts, every
    # m-tile width (16, 32, 64, 128 rows), with and without the shared expert
    (1, 256, 16, 1, 2, 256, 0),
    (37, 256, 16, 1, 4, 128, 1),
    (64, 512, 32, 0, 2, 256, 2),
    (200, 256, 16, 1, 2, 128, 3),
    (300, 256, 16, 1, 3, 256, 4),
    (700, 512, 16, 1, 2, 384, 5),
    # more than 96 rows per expert (several 128-row tiles per group): an odd number of
    # down K blocks (d_ff 384), a one-block down K (d_ff 128)
    (900, 256, 16, 1, 2, 384, 6),
    (2000, 256, 16, 0, 1, 128, 9),
]


# Twelve mixed shapes (drawn once from a seeded generator, then frozen): every
# m-tile width, d_model 256/512/768 (3-block down chunks), 16-64 experts,
# top-1..8, d_ff 128-512, with and without the shared expert.
MIXED = [
    (7, 768, 16, 0, 2, 256, 100),
    (777, 768, 64, 0, 8, 128, 101),
    (777, 256, 16, 0, 2, 512, 102),
    (7, 256, 32, 1, 5, 512, 103),
    (1500, 256, 32, 0, 5, 384, 104),
    (3, 512, 16, 1, 8, 384, 105),
    (64, 512, 32, 0, 3, 128, 106),
    (250, 512, 64, 1, 3, 384, 107),
    (511, 256, 32, 1, 3, 512, 108),
    (33, 256, 16, 0, 3, 128, 109),
    (511, 512, 64, 1, 3, 256, 110),
    (129, 256, 32, 0, 7, 256, 111),
]


@pytest.mark.parametrize("T,d,E,S,k,I,seed", SMALL + MIXED)
def test_small_fp8_layer(T, d, E, S, k, I, seed):
    _log(f"small fp8 T={T} d={d} E={E} S={S} k={k} I={I}")
    shape = synth.small_fp8(tokens=T, d_model=d, n_experts=E, n_shared=S, top_k=k, d_ff=I)
    inp = synth.generate(shape, seed=seed, device="cuda")
    g = gpu_chain(_layer(inp), inp)
    check_layer(inp, g)


@pytest.mark.parametrize("T,d,I,seed", [(9, 16384, 256, 11), (3, 256, 65536, 12)])
def test_small_fp8_largest_k(T, d, I, seed):
    """The largest supported contraction lengths: d_model 16384 (gate/up K
    = 128 blocks) and d_ff 65536 (down K = 512 blocks, the scale table's
    capacity)."""
    _log(f"largest K: T={T} d={d} I={I}")
    shape = synth.small_fp8(tokens=T, d_model=d, n_experts=16, n_shared=0, top_k=1, d_ff=I)
    inp = synth.generate(shape, seed=seed, device="cuda")
    g = gpu_chain(_layer(inp), inp)
    check_layer(inp, g)


@pytest.mark.parametrize("T", [333, 800])
def test_small_fp8_one_hot_expert_spans_many_tiles(T):
    # a large bias forces every token onto experts 3 and 11: m = T rows each,
    # several m-tiles per expert and the other experts empty (64- and 128-row
    # tiles)
    i, j = 3, 11
    shape = synth.small_fp8(tokens=T, n_experts=16, top_k=2, d_ff=256)
    inp = synth.generate(shape, seed=7, device="cuda")
    inp.bias[i] = 5.0
    inp.bias[j] = 5.0
    g = gpu_chain(_layer(inp), inp)
    assert np.all(g["ids"] == np.array([i, j]))
    check_layer(inp, g)


@pytest.mark.parametrize("T", [150, 40])   # 40 tokens: the one-workgroup permutation path
def test_small_dense_ffn(T):
    shape = synth.MoEShape("dense_small", tokens=T, d_model=256, n_experts=1, n_shared=0,
                           top_k=1, d_ff=384, fmt="fp8", routed_scaling=1.0, dense=True)
    inp = synth.generate(shape, seed=8, device="cuda")
    g = gpu_chain(_layer(inp), inp)
    check_layer(inp, g)


def test_quantiser_codes_over_wide_range():
    # columns scaled over 2^-20 .. 2^10 (RMSNorm keeps the spread inside a row),
    # so many codes are subnormal and every 1x128 block has a different scale
    shape = synth.small_fp8(tokens=96, n_experts=16, top_k=2)
    inp = synth.generate(shape, seed=9, device="cuda")
    scale = torch.logspace(-20, 10, shape.d_model, base=2.0, device="cuda")[None, :]
    inp.x = (inp.x.float() * scale).to(torch.bfloat16)
    inp.x[5, :128] = 0               # an all-zero 1x128 block in one token
    g = gpu_chain(_layer(inp), inp)
    ref = run_oracle(inp, tokens=np.arange(96), ids_override=g["ids"])
    assert np.array_equal(g["xs"], ref["xs"])
    assert np.array_equal(g["xq"], ref["xq"])


def test_zero_tokens_and_determinism():
    shape = synth.small_fp8(tokens=50, n_experts=16, top_k=4)
    inp = synth.generate(shape, seed=10, device="cuda")
    layer = _layer(inp)
    empty = layer.forward(inp.x[:0])
    assert empty.shape == (0, shape.d_model)
    a = layer.forward(inp.x).clone()
    b = layer.forward(inp.x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------- K2 shapes
@pytest.fixture(scope="module")
def k2():
    _log("generating K2 weights on the GPU")
    base = synth.generate(synth.K2_DECODE, seed=0, device="cuda")
    layer = _layer(base)
    _log("packed")
    return base, layer


def _sample(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(n, T), replace=False))


def test_k2_decode(k2):
    base, layer = k2
    inp = base
    g = gpu_chain(layer, inp)
    _log(f"decode: touched experts {int(np.sum(np.diff(g['offsets']) > 0))}")
    check_layer(inp, g, tokens=_sample(64, 8))


def test_k2_prefill(k2):
    base, layer = k2
    inp = synth.with_workload(base, synth.K2_PREFILL, seed=0)
    g = gpu_chain(layer, inp)
    counts = np.diff(g["offsets"])
    _log(f"prefill: tokens per expert min {counts.min()} max {counts.max()}")
    check_layer(inp, g, tokens=_sample(8192, 4, seed=1))
    a = layer.forward(inp.x).clone()
    torch.cuda.synchronize()
    assert np.array_equal(to_f32(a).view(np.uint32), g["out_f"].view(np.uint32))


def test_k2_skewed(k2):
    base, layer = k2
    inp = synth.with_workload(base, synth.K2_SKEWED, seed=0)
    g = gpu_chain(layer, inp)
    counts = np.diff(g["offsets"])
    hot = int(np.argmax(counts))
    _log(f"skewed: max {counts.max()} (expert {hot}), experts under 10 tokens "
         f"{int(np.sum(counts < 10))}, empty {int(np.sum(counts == 0))}")
    hot_tok = int(g["row_pair"][g["offsets"][hot]] // 8)
    toks = np.unique(np.concatenate([_sample(16384, 3, seed=2), [hot_tok]]))
    check_layer(inp, g, tokens=toks)


@pytest.mark.parametrize("T", [1, 5, 257, 700, 1000, 2000, 3000, 5000])
def test_k2_ragged_token_counts(k2, T):
    """K2 dimensions at token counts that select every m-tile width (16, 32,
    64 and 128 rows) and leave ragged last tiles in most experts."""
    base, layer = k2
    inp = synth.with_workload(base, synth.K2_DECODE, seed=100 + T, tokens=T)
    g = gpu_chain(layer, inp)
    counts = np.diff(g["offsets"])
    _log(f"T={T}: mean rows per routed expert {T * 8 / 384:.1f}, max {counts.max()}")
    check_layer(inp, g, tokens=_sample(T, 3, seed=T))


def test_k2_maximum_token_count(k2):
    """The largest batch one call accepts at the K2 shape: T (top_k + 1)
    max(d_model, d_ff) < 2^32 gives 66,576 tokens (1,041 permutation chunks,
    599,184 GEMM rows); one more is rejected on the host."""
    base, layer = k2
    T = 66576
    inp = synth.with_workload(base, synth.K2_DECODE, seed=4242, tokens=T)
    g = gpu_chain(layer, inp)
    counts = np.diff(g["offsets"])
    _log(f"T={T}: rows per routed expert min {counts.min()} max {counts.max()}")
    toks = np.unique(np.concatenate([_sample(T, 3, seed=5), [0, T - 1]]))
    check_layer(inp, g, tokens=toks)


@pytest.mark.parametrize("workload", ["decode", "prefill"])
def test_k2_repeats_with_poisoned_buffers(k2, workload):
    """Ten forwards with the workspace and the output filled with 0xFF bytes
    (NaN in every float view, -1 in every index view) before each call are
    bitwise equal to a clean run: nothing is read before it is written."""
    from sparse_moe_transformer_sigmoid_amd import _lib as L
    base, layer = k2
    inp = base if workload == "decode" else synth.with_workload(base, synth.K2_PREFILL, seed=0)
    layer.use_router(inp)
    x = inp.x
    ref = layer.forward(x).clone()
    ws = layer.workspace(x.shape[0], L.MOE_WS_FORWARD)
    out = torch.empty_like(ref)
    for r in range(10):
        ws.fill_(0xFF)
        out.view(torch.int16).fill_(-1)
        layer.forward(x, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"run {r}"
    _log(f"{workload}: 10 poisoned runs bitwise equal")


def test_k2_decode_graph_replay(k2):
    """moe_forward captured in a HIP graph: every replay equals the eager call,
    with eager work on other inputs and synchronisations between replays."""
    base, layer = k2
    layer.use_router(base)
    x = base.x
    eager = layer.forward(x).clone()
    other = torch.flip(x, dims=[0]).contiguous()
    out = torch.empty_like(eager)
    g = layer.capture_forward(x, out)
    for r in range(3):
        out.zero_()
        layer.forward(other)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _log(f"graph replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
    del g


def test_k2_ep8_shard():
    """One GPU's share under 8-way expert parallelism: 48 experts with about
    1365 rows each (eleven 128-row tiles per expert)."""
    inp = synth.generate(synth.K2_EP8_SHARD, seed=0, device="cuda")
    layer = _layer(inp)
    g = gpu_chain(layer, inp)
    counts = np.diff(g["offsets"])
    _log(f"ep8 shard: rows per expert min {counts.min()} max {counts.max()}")
    check_layer(inp, g, tokens=_sample(8192, 3, seed=4))
    del layer


def test_k2_dense_ffn():
    inp = synth.generate(synth.K2_DENSE, seed=0, device="cuda")
    layer = _layer(inp)
    g = gpu_chain(layer, inp)
    check_layer(inp, g, tokens=_sample(4096, 3, seed=3))
    del layer
