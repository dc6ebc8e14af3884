"""ctypes binding of libk2moe.so: the C ABI in include/k2moe.h and include/k2mla.h,
same names.

Argument marshalling only -- every step of the layer runs in the HIP
library.  Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

from .build import lib_path

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_FMT_F32, MOE_FMT_BF16_FP8B128 = 0, 1
MOE_WS_ROUTER, MOE_WS_PERMUTE, MOE_WS_SWIGLU, MOE_WS_FORWARD = range(4)


class moe_config(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_experts", C.c_int32), ("n_shared", C.c_int32),
                ("top_k", C.c_int32), ("d_ff", C.c_int32), ("n_group", C.c_int32),
                ("topk_group", C.c_int32), ("norm_topk_prob", C.c_int32), ("fmt", C.c_int32),
                ("dense", C.c_int32), ("routed_scaling", C.c_float), ("rms_eps", C.c_float)]


class moe_expert_w(C.Structure):
    _fields_ = [("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

class mla_config(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_heads", C.c_int32), ("q_lora", C.c_int32),
                ("kv_lora", C.c_int32), ("qk_nope", C.c_int32), ("qk_rope", C.c_int32),
                ("v_head", C.c_int32), ("rope_orig_len", C.c_int32), ("rope_theta", C.c_float),
                ("rope_factor", C.c_float), ("beta_fast", C.c_float), ("beta_slow", C.c_float),
                ("mscale_all_dim", C.c_float), ("rms_eps", C.c_float)]


class mla_weights(C.Structure):
    _fields_ = [("w_qa", C.c_void_p), ("s_qa", C.c_void_p), ("w_qb", C.c_void_p),
                ("s_qb", C.c_void_p), ("w_kva", C.c_void_p), ("s_kva", C.c_void_p),
                ("w_kvb", C.c_void_p), ("s_kvb", C.c_void_p), ("w_o", C.c_void_p),
                ("s_o", C.c_void_p), ("g_qa", C.c_void_p), ("g_kva", C.c_void_p)]


EXPORTS = ["moe_status_str", "moe_last_error", "moe_packed_weights_bytes", "moe_pack_weights",
           "moe_workspace_bytes", "moe_router", "moe_permute", "moe_grouped_swiglu",
           "moe_combine", "moe_forward", "moe_profile_enable", "moe_profile_read",
           "mla_packed_weights_bytes", "mla_pack_weights", "mla_workspace_bytes", "mla_forward",
           "mla_attention", "moe_forward_noalloc", "moe_expert_load", "moe_bias_update",
           "moe_train_weights_bytes", "moe_train_transposed_bytes", "moe_train_transpose_weights",
           "moe_train_saved_bytes", "moe_train_workspace_bytes", "moe_train_forward",
           "moe_train_backward"]
STAGES = ["norm_quant", "router_gemm", "topk", "permute", "tiles", "gateup", "down", "combine",
          "mla_proj", "mla_latent", "mla_attn", "mla_vup", "balance", "train_fwd", "train_dgrad",
          "train_wgrad", "train_other"]

_LIB = None


def load(path: str | None = None) -> C.CDLL:
    """Load libk2moe.so (raises if it is missing: there is no fallback)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or lib_path()
    if not os.path.exists(p):
        raise ImportError(f"{p} not built; run python -m sparse_moe_transformer_sigmoid_amd.build")
    lib = C.CDLL(p)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    cfgp = C.POINTER(moe_config)
    sig = {
        "moe_status_str": (C.c_char_p, [i32]),
        "moe_last_error": (C.c_char_p, []),
        "moe_packed_weights_bytes": (sz, [cfgp]),
        "moe_pack_weights": (i32, [cfgp, C.POINTER(moe_expert_w), i32, vp, vp]),
        "moe_workspace_bytes": (i32, [cfgp, i64, i32, C.POINTER(sz)]),
        "moe_router": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_permute": (i32, [cfgp, i64, vp, vp, vp, vp, vp, sz, vp]),
        "moe_grouped_swiglu": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                     vp]),
        "moe_combine": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, i32, vp]),
        "moe_forward": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_profile_enable": (i32, [i32]),
        "moe_profile_read": (i32, [C.POINTER(C.c_double), C.POINTER(C.c_int64), i32]),
        "moe_forward_noalloc": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp]),
        "moe_expert_load": (i32, [cfgp, i64, vp, vp, vp]),
        "moe_bias_update": (i32, [cfgp, vp, C.c_float, vp, vp]),
        "moe_train_weights_bytes": (sz, [cfgp]),
        "moe_train_transposed_bytes": (sz, [cfgp]),
        "moe_train_transpose_weights": (i32, [cfgp, vp, vp, vp]),
        "moe_train_saved_bytes": (i32, [cfgp, i64, C.POINTER(sz)]),
        "moe_train_workspace_bytes": (i32, [cfgp, i64, C.POINTER(sz)]),
        "moe_train_forward": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_train_backward": (i32, [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]),
        "mla_packed_weights_bytes": (sz, [C.POINTER(mla_config)]),
        "mla_pack_weights": (i32, [C.POINTER(mla_config), C.POINTER(mla_weights), vp, vp]),
        "mla_workspace_bytes": (i32, [C.POINTER(mla_config), i32, i32, i32, C.POINTER(sz)]),
        "mla_forward": (i32, [C.POINTER(mla_config), i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                              vp, i32, vp, sz, vp]),
        "mla_attention": (i32, [C.POINTER(mla_config), i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status, load().moe_last_error().decode())


def call(fn: str, *args) -> None:
    """Call an ABI entry point and raise MoEError on a non-OK status."""
    check(fn, getattr(load(), fn)(*args))


def status_of(fn: str, *args) -> int:
    """Call an ABI entry point and return its raw status."""
    return getattr(load(), fn)(*args)
