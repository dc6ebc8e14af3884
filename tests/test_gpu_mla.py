"""Parity of the MLA attention sub-layer (through the C ABI) with the CPU oracle.

Small layers are compared on every token; the Kimi K2 shapes (64-sequence
decode over 4,096 cached positions, 2 x 4,096-token prefill) run whole on the
GPU in the launch configuration the benchmark times and are compared on
sampled tokens (every new cache entry at decode).  The oracle evaluates the
definition: per-head keys and values from the cached latent, exact sums.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_ref as R
from oracle.adapt import run_mla_oracle, to_f32
from oracle.compare import close_report

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


def gpu_run(inp, layer=None):
    from sparse_moe_transformer_sigmoid_amd.mla import K2MLA
    sh = inp.shape
    layer = layer or K2MLA(inp)
    c1 = inp.fresh_cache()
    y = layer.forward(inp.x, inp.cached_len, c1, sh.n_seq, sh.n_new, out_f32=True)
    c2 = inp.fresh_cache()
    out = layer.forward(inp.x, inp.cached_len, c2, sh.n_seq, sh.n_new)
    c3 = inp.fresh_cache()
    attn = layer.attention(inp.x, inp.cached_len, c3, sh.n_seq, sh.n_new)
    torch.cuda.synchronize()
    for a, b in zip(c1, c2):        # the three calls write the same cache entries
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    for a, b in zip(c1, c3):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    return dict(y=y.cpu().numpy(), out=to_f32(out), attn=attn.cpu().numpy(),
                codes=c1[0].cpu().numpy(), scales=c1[1].cpu().numpy(), rope=to_f32(c1[2]))


def _gate(gpu, ref, what, bf16_out=False):
    rep = close_report(gpu, ref, bf16_out=bf16_out)
    _log(f"  {what}: max_abs/rms {rep['max_abs'] / max(rep['rms'], 1e-30):.3e} "
         f"mean_rel {rep['mean_rel']:.3e} ok {rep['ok']}")
    assert rep["ok"], f"{what}: {rep}"
    return rep


def check_cache(g, ref):
    """New cache entries: the latent's codes within one e4m3 step of the
    oracle's and its scales within 1% (both are decisions on the projected,
    normalised latent), the rotated positional key within the tolerance."""
    seq, pos = ref["seq_of"], ref["pos_of"]
    gc, rc = g["codes"][seq, pos], ref["cache"]["codes"][seq, pos]
    gs, rs = g["scales"][seq, pos], ref["cache"]["scales"][seq, pos]
    same = float(np.mean(gc == rc))
    srel = float(np.max(np.abs(gs.astype(np.float64) / rs - 1.0)))
    dg = R.dequantize_1x128(gc, rs)
    dr = R.dequantize_1x128(rc, rs)
    step = np.abs(dr) * 2.0 ** -3
    amax = np.repeat(rs.astype(np.float64) * 448.0, 128, axis=1)
    excess = float((np.abs(dg - dr) - np.maximum(step, 2e-3 * amax)).max())
    _log(f"  cache latent codes equal {same:.4f}, worst excess over one step {excess:.2e}, "
         f"scale rel diff {srel:.2e}")
    assert excess <= 0 and srel <= 1e-2 and same >= 0.9
    _gate(g["rope"][seq, pos], ref["cache"]["rope"][seq, pos], "cache rotary keys")
    # positions outside the new ones are untouched
    mask = np.ones(g["codes"].shape[:2], dtype=bool)
    mask[seq, pos] = False
    assert np.array_equal(g["codes"][mask], ref["cache"]["codes"][mask])


def check_mla(inp, tokens=None):
    g = gpu_run(inp)
    ref = run_mla_oracle(inp, tokens=tokens)
    sel = ref["tokens"]
    check_cache(g, ref)
    _gate(g["attn"][sel], ref["o"], "attention output (W_o input)")
    _gate(g["y"][sel], ref["y"], "y = W_o attention")
    _gate(g["out"][sel], ref["out"], "out", bf16_out=True)
    return g, ref


# ------------------------------------------------------------- small layers
@pytest.mark.parametrize("n_seq,n_new,cached,max_len,heads,seed", [
    (3, 1, (0, 5, 300), 320, 16, 0),           # decode, ragged lengths, an empty prefix
    (4, 1, (1, 100, 1000, 2047), 2048, 64, 1),  # decode with 64 heads: one token per workgroup
    (2, 37, (0, 20), 64, 16, 2),                # prefill: 4-token blocks with a ragged tail
    (1, 64, (0,), 64, 64, 3),                   # prefill with 64 heads
    (2, 5, (300, 0), 400, 32, 4),               # chunked prefill after a cached prefix
])
def test_small_mla(n_seq, n_new, cached, max_len, heads, seed):
    _log(f"small mla S={n_seq} n={n_new} cached={cached} L={max_len} H={heads}")
    shape = synth.small_mla(n_seq=n_seq, n_new=n_new, cached=cached, max_len=max_len,
                            n_heads=heads, d_model=512 if heads <= 32 else 256)
    inp = synth.generate_mla(shape, seed=seed, device="cuda")
    check_mla(inp)


def _edge_tokens(n_seq, n_new):
    """Per sequence: the first and last new token, both ends of every 32-token
    wave block and of every 256-token workgroup tile, and the middle."""
    local = {0, n_new - 1, n_new // 2}
    for b in range(0, n_new, 32):
        local.update((b, min(b + 31, n_new - 1)))
    return np.array(sorted(s * n_new + i for s in range(n_seq) for i in local if i < n_new))


# Prompt-sized batches (>= 128 new tokens per sequence) attend in the per-head
# form (keys and values formed per position and head, flash-style attention).
@pytest.mark.parametrize("n_seq,n_new,cached,max_len,heads,seed", [
    (2, 128, (0, 37), 192, 16, 10),             # the smallest such batch, one cached prefix
    (1, 300, (0,), 320, 64, 11),                # 64 heads, a ragged second 256-token tile
    (2, 150, (500, 3), 700, 32, 12),            # chunked prefill after a long prefix; idle waves
    (3, 129, (64, 0, 31), 224, 16, 13),         # ragged lengths, a 64-position-aligned prefix
    (2, 1024, (0, 100), 1200, 16, 14),          # 2,048 tokens: the output projection in 128-row tiles
])
def test_small_mla_per_head_form(n_seq, n_new, cached, max_len, heads, seed):
    _log(f"per-head mla S={n_seq} n={n_new} cached={cached} L={max_len} H={heads}")
    shape = synth.small_mla(n_seq=n_seq, n_new=n_new, cached=cached, max_len=max_len,
                            n_heads=heads, d_model=512 if heads <= 32 else 256)
    inp = synth.generate_mla(shape, seed=seed, device="cuda")
    check_mla(inp, tokens=_edge_tokens(n_seq, n_new))


def test_small_mla_random_gamma():
    shape = synth.small_mla(n_seq=2, n_new=3, cached=(7, 40), max_len=64, gamma_std=0.1)
    inp = synth.generate_mla(shape, seed=5, device="cuda")
    assert float(inp.g_kva.float().std()) > 0.05
    check_mla(inp)


def test_small_mla_deterministic_and_zero_tokens():
    from sparse_moe_transformer_sigmoid_amd.mla import K2MLA
    shape = synth.small_mla(n_seq=2, n_new=9, cached=(3, 50), max_len=80)
    inp = synth.generate_mla(shape, seed=6, device="cuda")
    layer = K2MLA(inp)
    a = gpu_run(inp, layer)
    b = gpu_run(inp, layer)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    empty = layer.forward(inp.x[:0], inp.cached_len, inp.fresh_cache(), 0, 9)
    assert empty.shape[0] == 0


# -------------------------------------------------------------- K2 shapes
def test_k2_mla_decode():
    """64 sequences x 4,096 cached positions, one new token each."""
    inp = synth.generate_mla(synth.MLA_K2_DECODE, seed=0, device="cuda")
    check_mla(inp, tokens=np.array([0, 9, 31, 63]))


def test_k2_mla_decode_graph_replay():
    """mla_forward captured in a HIP graph: every replay equals the eager call
    bitwise (output and new cache entries), with eager work on other inputs and
    synchronisations between replays."""
    from sparse_moe_transformer_sigmoid_amd.mla import K2MLA
    inp = synth.generate_mla(synth.MLA_K2_DECODE, seed=0, device="cuda")
    layer = K2MLA(inp)
    S, n = inp.shape.n_seq, inp.shape.n_new
    pos = inp.cached_len.long()                 # the new token's position per sequence
    seqs = torch.arange(S, device=pos.device)
    cache = inp.fresh_cache()
    eager = layer.forward(inp.x, inp.cached_len, cache, S, n).clone()
    eager_cache = [c.clone() for c in cache]
    other_x = torch.flip(inp.x, dims=[0]).contiguous()
    other_cache = inp.fresh_cache()
    out = torch.empty_like(eager)
    g = layer.capture_forward(inp.x, inp.cached_len, cache, S, n, out)
    for r in range(3):
        out.zero_()
        for c in cache:
            c[seqs, pos] = 0                    # the replay must write them again
        layer.forward(other_x, inp.cached_len, other_cache, S, n)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _log(f"mla graph replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        # the replay rewrites only the new positions: compare those entries
        for c, e in zip(cache, eager_cache):
            assert torch.equal(c[seqs, pos].view(torch.uint8), e[seqs, pos].view(torch.uint8)), \
                f"replay {r}: cache entries"
    del g


def test_k2_mla_prefill():
    """2 x 4,096 new tokens from an empty cache; tokens at the start, the middle
    and the end of both sequences."""
    inp = synth.generate_mla(synth.MLA_K2_PREFILL, seed=0, device="cuda")
    check_mla(inp, tokens=np.array([0, 1, 2047, 4095, 4096 + 100, 8191]))
