"""PyTorch-side wrapper of the training-step entry points (include/k2train.h).

torch allocates the buffers and supplies the stream; each method marshals
pointers into ABI calls.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L
from .layer import config_from_shape


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class K2Train:
    """One MoE layer's training step with bf16 weights resident on the GPU."""

    def __init__(self, inputs, device="cuda"):
        self.shape = inputs.shape
        self.cfg = config_from_shape(self.shape)
        self.device = torch.device(device)
        self.norm_w, self.w_router, self.bias = inputs.norm_w, inputs.w_router, inputs.bias
        self.w = inputs.w
        lib = L.load()
        n = lib.moe_train_transposed_bytes(C.byref(self.cfg))
        if n == 0:
            raise L.MoEError("moe_train_transposed_bytes", L.MOE_ERR_INVALID_ARG,
                             lib.moe_last_error().decode())
        self.wt = torch.empty(n, dtype=torch.uint8, device=self.device)
        self.transpose_weights()
        self._ws = {}

    def transpose_weights(self):
        """moe_train_transpose_weights: refresh the transposed copies from self.w."""
        L.call("moe_train_transpose_weights", C.byref(self.cfg), _p(self.w), _p(self.wt),
               _stream())

    def _size(self, fn, T):
        n = C.c_size_t(0)
        L.call(fn, C.byref(self.cfg), T, C.byref(n))
        return max(n.value, 256)

    def workspace(self, T):
        if T not in self._ws:
            self._ws[T] = torch.empty(self._size("moe_train_workspace_bytes", T),
                                      dtype=torch.uint8, device=self.device)
        return self._ws[T]

    def saved_buffer(self, T):
        return torch.empty(self._size("moe_train_saved_bytes", T), dtype=torch.uint8,
                           device=self.device)

    def forward(self, x, saved=None, out=None):
        """out [T, d] bf16 and the saved state (a byte buffer) for the backward."""
        T = x.shape[0]
        saved = self.saved_buffer(T) if saved is None else saved
        out = torch.empty_like(x) if out is None else out
        ws = self.workspace(T)
        L.call("moe_train_forward", C.byref(self.cfg), T, _p(x), _p(self.norm_w),
               _p(self.w_router), _p(self.bias), _p(self.w), _p(out), _p(saved), _p(ws),
               ws.numel(), _stream())
        return out, saved

    def backward(self, dout, x, saved, grads=None, dh_rows=False, dw=False):
        """Gradients (fp32): dict dx, d_norm_w, d_w_router, d_w (canonical
        layout), and optionally dh_rows [R, d] and dw [T, k]."""
        sh = self.shape
        T, d = x.shape
        G = sh.n_experts + sh.n_shared
        f = dict(dtype=torch.float32, device=self.device)
        g = grads or {"dx": torch.empty((T, d), **f), "d_norm_w": torch.empty(d, **f),
                      "d_w_router": torch.empty((sh.n_experts, d), **f),
                      "d_w": torch.empty(G * 3 * sh.d_ff * d, **f)}
        if dh_rows and "dh_rows" not in g:
            g["dh_rows"] = torch.empty((T * sh.top_k + T * sh.n_shared, d), **f)
        if dw and "dw" not in g:
            g["dw"] = torch.empty((T, sh.top_k), **f)
        ws = self.workspace(T)
        L.call("moe_train_backward", C.byref(self.cfg), T, _p(dout), _p(x), _p(self.norm_w),
               _p(self.w_router), _p(self.w), _p(self.wt), _p(saved), _p(g["dx"]),
               _p(g["d_norm_w"]), _p(g["d_w_router"]), _p(g["d_w"]), _p(g.get("dh_rows")),
               _p(g.get("dw")), _p(ws), ws.numel(), _stream())
        return g
