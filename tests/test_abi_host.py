"""Host-side checks of the C ABI: symbols, sizes and argument validation.

Runs without a GPU.  Every call here either fails validation or has T = 0,
so the library returns before making any HIP call.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

import synth
from sparse_moe_transformer_sigmoid_amd import _lib as L
from sparse_moe_transformer_sigmoid_amd.build import lib_path
from sparse_moe_transformer_sigmoid_amd.layer import config_from_shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("k2moe.h", "k2mla.h", "k2train.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(lib_path()),
                                reason="libk2moe.so not built")

FAKE = 0x10000          # aligned non-null stand-in; never dereferenced (validation fails first)


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:moe|mla)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(
        os.path.basename(h) for h in HEADERS)


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(L.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT ((?:moe|mla)_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = L.load()
    for n in names:
        assert getattr(lib, n) is not None


def _cfg(shape=synth.K2_DECODE, **kw):
    c = config_from_shape(shape)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_status_strings():
    lib = L.load()
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(3) == b"MOE_ERR_WORKSPACE"


def test_packed_bytes_match_page_expert_size():
    lib = L.load()
    cfg = _cfg()
    n = lib.moe_packed_weights_bytes(C.byref(cfg))
    per_expert = 3 * 2048 * 7168          # 44,040,192 FP8 weights per expert
    assert per_expert == 44_040_192
    scales = 385 * (16 * 56 * 2 + 56 * 16) * 4
    assert 385 * per_expert + scales <= n < 385 * per_expert + scales + 3 * 256
    bad = _cfg(n_group=2)
    assert lib.moe_packed_weights_bytes(C.byref(bad)) == 0


def test_workspace_sizes_monotone_in_tokens():
    cfg = _cfg()
    sizes = []
    for T in (0, 1, 64, 8192):
        n = C.c_size_t()
        L.call("moe_workspace_bytes", C.byref(cfg), T, L.MOE_WS_FORWARD, C.byref(n))
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[-1] > 8192 * 8 * 7168 * 4


@pytest.mark.parametrize("field,value,status", [
    ("n_group", 2, L.MOE_ERR_UNSUPPORTED),
    ("topk_group", 4, L.MOE_ERR_UNSUPPORTED),
    ("fmt", 7, L.MOE_ERR_UNSUPPORTED),
    ("top_k", 0, L.MOE_ERR_INVALID_ARG),
    ("top_k", 385, L.MOE_ERR_INVALID_ARG),
    ("n_shared", 2, L.MOE_ERR_UNSUPPORTED),
    ("d_model", 7168 + 128, L.MOE_ERR_UNSUPPORTED),
    ("d_ff", 2048 + 64, L.MOE_ERR_UNSUPPORTED),
    ("n_experts", 392 + 4, L.MOE_ERR_UNSUPPORTED),
    ("dense", 1, L.MOE_ERR_INVALID_ARG),
])
def test_config_validation(field, value, status):
    cfg = _cfg(**{field: value})
    n = C.c_size_t()
    assert L.status_of("moe_workspace_bytes", C.byref(cfg), 8, 0, C.byref(n)) == status
    assert L.load().moe_last_error()


def _forward_args(cfg, T=4, ws_bytes=1 << 40, **over):
    args = dict(x=FAKE, norm_w=FAKE, w_router=FAKE, bias=FAKE, packed=FAKE, out=FAKE, ws=FAKE)
    args.update(over)
    return (C.byref(cfg), T, args["x"], args["norm_w"], args["w_router"], args["bias"],
            args["packed"], args["out"], args["ws"], ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "norm_w", "w_router", "bias", "packed", "out", "ws"])
def test_forward_rejects_null_pointer(name):
    cfg = _cfg()
    assert L.status_of("moe_forward", *_forward_args(cfg, **{name: None})) == L.MOE_ERR_INVALID_ARG


def test_forward_rejects_misaligned_pointer():
    cfg = _cfg()
    assert L.status_of("moe_forward", *_forward_args(cfg, x=FAKE + 2)) == L.MOE_ERR_INVALID_ARG


def test_forward_small_workspace_and_negative_tokens():
    cfg = _cfg()
    n = C.c_size_t()
    L.call("moe_workspace_bytes", C.byref(cfg), 64, L.MOE_WS_FORWARD, C.byref(n))
    assert L.status_of("moe_forward", *_forward_args(cfg, T=64, ws_bytes=n.value - 1)) == \
        L.MOE_ERR_WORKSPACE
    assert L.status_of("moe_forward", *_forward_args(cfg, T=-1)) == L.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op():
    cfg = _cfg()
    assert L.status_of("moe_forward", *_forward_args(cfg, T=0, ws_bytes=0)) == L.MOE_OK
    # empty tensors may have null data pointers
    assert L.status_of("moe_forward", *_forward_args(cfg, T=0, ws_bytes=0, x=None, out=None,
                                                     ws=None)) == L.MOE_OK
    assert L.status_of("moe_permute", C.byref(cfg), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                       None) == L.MOE_OK


def test_dense_mode_allows_missing_router():
    cfg = _cfg(synth.K2_DENSE)
    assert L.status_of("moe_forward", *_forward_args(cfg, T=0, w_router=None, bias=None,
                                                     ws_bytes=0)) == L.MOE_OK
    cfg2 = _cfg()
    assert L.status_of("moe_forward", *_forward_args(cfg2, T=4, w_router=None)) == \
        L.MOE_ERR_INVALID_ARG


def test_router_f32_requires_null_scales():
    cfg = _cfg(synth.TINY)
    st = L.status_of("moe_router", C.byref(cfg), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                     FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == L.MOE_ERR_INVALID_ARG


def test_swiglu_shared_out_must_match_config():
    cfg = _cfg()
    st = L.status_of("moe_grouped_swiglu", C.byref(cfg), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                     None, None, None, FAKE, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG
    st = L.status_of("moe_grouped_swiglu", C.byref(cfg), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                     FAKE, FAKE, None, FAKE, 1 << 40, None)     # act_q without act_s
    assert st == L.MOE_ERR_INVALID_ARG


def test_pack_rejects_wrong_expert_count():
    cfg = _cfg(synth.TINY)
    arr = (L.moe_expert_w * 3)()
    assert L.status_of("moe_pack_weights", C.byref(cfg), arr, 3, FAKE, None) == \
        L.MOE_ERR_INVALID_ARG


# ---- MLA attention entry points (include/k2mla.h)
def _mla_cfg(**kw):
    from sparse_moe_transformer_sigmoid_amd.mla import mla_config_from_shape
    c = mla_config_from_shape(synth.MLA_K2_DECODE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_mla_sizes_and_validation():
    lib = L.load()
    cfg = _mla_cfg()
    # packed: the three GEMM matrices as FP8 codes (the stacked
    # down-projections padded to 2304 rows), the key-value up-projection as
    # bf16 copies (2 bytes per weight; the key rows twice, transposed and as
    # they are), scales, norms and frequencies
    n = lib.mla_packed_weights_bytes(C.byref(cfg))
    fp8 = 2304 * 7168 + 12288 * 1536 + 7168 * 8192
    bf16 = 2 * (16384 + 8192) * 512
    assert fp8 + bf16 < n < (fp8 + bf16) * 1.01
    nb = C.c_size_t(0)
    assert lib.mla_workspace_bytes(C.byref(cfg), 64, 1, 4097, C.byref(nb)) == L.MOE_OK
    assert nb.value > 64 * 12288 * 4
    decode = nb.value
    assert lib.mla_workspace_bytes(C.byref(cfg), 0, 1, 4097, C.byref(nb)) == L.MOE_OK
    assert nb.value == 0
    # prompt-sized batches (>= 128 new tokens per sequence) attend in the
    # per-head form: keys and values of every position and head as bf16
    # high/low halves, 1 KiB per (position, head), and no absorbed queries
    # (64 x 576 fp32 per token); below that, the absorbed form's buffers
    kv = 2 * 64 * 4096 * 1024
    qcat = 64 * 576 * 4
    assert lib.mla_workspace_bytes(C.byref(cfg), 2, 4096, 4096, C.byref(nb)) == L.MOE_OK
    assert kv < nb.value < kv + 2 * 4096 * qcat
    assert lib.mla_workspace_bytes(C.byref(cfg), 2, 127, 4096, C.byref(nb)) == L.MOE_OK
    assert 2 * 127 * qcat < nb.value < kv
    assert decode < kv
    for bad in (dict(kv_lora=256), dict(qk_rope=32), dict(n_heads=24), dict(d_model=7000)):
        c = _mla_cfg(**bad)
        assert lib.mla_packed_weights_bytes(C.byref(c)) == 0
        assert lib.mla_workspace_bytes(C.byref(c), 1, 1, 16, C.byref(nb)) == \
            L.MOE_ERR_UNSUPPORTED, bad
    assert lib.mla_workspace_bytes(C.byref(cfg), 1, 20, 16, C.byref(nb)) == L.MOE_ERR_INVALID_ARG
    assert lib.mla_workspace_bytes(C.byref(cfg), -1, 1, 16, C.byref(nb)) == L.MOE_ERR_INVALID_ARG


def test_mla_forward_argument_checks():
    lib = L.load()
    cfg = _mla_cfg()
    p = [FAKE] * 7
    # T = 0: nothing is examined or enqueued
    st = lib.mla_forward(C.byref(cfg), 0, 1, 16, *[None] * 7, None, 0, None, 0, None)
    assert st == L.MOE_OK
    # a null input, a misaligned one, a small workspace, a bad flag
    st = lib.mla_forward(C.byref(cfg), 2, 1, 16, None, *p[1:], FAKE, 0, FAKE, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG and b"x is NULL" in lib.moe_last_error()
    st = lib.mla_forward(C.byref(cfg), 2, 1, 16, FAKE + 4, *p[1:], FAKE, 0, FAKE, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG and b"aligned" in lib.moe_last_error()
    st = lib.mla_forward(C.byref(cfg), 2, 1, 16, *p, FAKE, 0, FAKE, 16, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.mla_forward(C.byref(cfg), 2, 1, 16, *p, FAKE, 2, FAKE, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG
    st = lib.mla_attention(C.byref(cfg), 2, 1, 16, *p, None, FAKE, 1 << 40, None)
    assert st == L.MOE_ERR_INVALID_ARG and b"attn is NULL" in lib.moe_last_error()
    st = lib.mla_pack_weights(C.byref(cfg), None, FAKE, None)
    assert st == L.MOE_ERR_INVALID_ARG


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    """The static scratch array holds 48 MiB: 130 tokens at the K2 shape fit,
    131 do not (checked on the host, before any HIP call)."""
    lib = L.load()
    cfg = _cfg()
    n = C.c_size_t(0)
    assert lib.moe_workspace_bytes(C.byref(cfg), 130, L.MOE_WS_FORWARD, C.byref(n)) == L.MOE_OK
    assert n.value <= 48 << 20
    assert lib.moe_workspace_bytes(C.byref(cfg), 131, L.MOE_WS_FORWARD, C.byref(n)) == L.MOE_OK
    assert n.value > 48 << 20
    st = lib.moe_forward_noalloc(C.byref(cfg), 131, *[FAKE] * 7, None)
    assert st == L.MOE_ERR_WORKSPACE and b"50331648" in lib.moe_last_error()
    assert lib.moe_forward_noalloc(C.byref(cfg), 0, *[None] * 7, None) == L.MOE_OK


def test_balance_argument_checks():
    cfg = _cfg()
    nan, inf = float("nan"), float("inf")
    # loads: T < 0, NULL or misaligned arrays; T = 0 is a no-op
    assert L.status_of("moe_expert_load", C.byref(cfg), -1, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert L.status_of("moe_expert_load", C.byref(cfg), 4, None, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert L.status_of("moe_expert_load", C.byref(cfg), 4, FAKE, FAKE + 2, None) == \
        L.MOE_ERR_INVALID_ARG
    assert L.status_of("moe_expert_load", C.byref(cfg), 0, None, None, None) == L.MOE_OK
    # update: speed finite and >= 0, both arrays present and aligned
    for bad in (nan, inf, -1e-3):
        assert L.status_of("moe_bias_update", C.byref(cfg), FAKE, C.c_float(bad), FAKE, None) == \
            L.MOE_ERR_INVALID_ARG, bad
    assert L.status_of("moe_bias_update", C.byref(cfg), None, C.c_float(1e-3), FAKE, None) == \
        L.MOE_ERR_INVALID_ARG
    assert L.status_of("moe_bias_update", C.byref(cfg), FAKE, C.c_float(1e-3), FAKE + 1, None) == \
        L.MOE_ERR_INVALID_ARG
    # a dense layer has no routed experts and no bias
    dense = _cfg(synth.K2_DENSE)
    assert L.status_of("moe_expert_load", C.byref(dense), 4, FAKE, FAKE, None) == \
        L.MOE_ERR_INVALID_ARG
    assert L.status_of("moe_bias_update", C.byref(dense), FAKE, C.c_float(1e-3), FAKE, None) == \
        L.MOE_ERR_INVALID_ARG
    assert "dense" in L.load().moe_last_error().decode()
