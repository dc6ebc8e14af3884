"""PyTorch-side wrapper of the MLA attention entry points (include/k2mla.h).

torch allocates the buffers and supplies the stream; each method marshals
pointers into one ABI call.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L


def mla_config_from_shape(shape) -> L.mla_config:
    c = L.mla_config()
    for name, _ in L.mla_config._fields_:
        setattr(c, name, getattr(shape, name))
    return c


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class K2MLA:
    """One MLA attention sub-layer with packed weights resident on the GPU."""

    def __init__(self, inputs, device="cuda"):
        self.shape = inputs.shape
        self.cfg = mla_config_from_shape(self.shape)
        self.device = torch.device(device)
        self.norm_w = inputs.norm_w
        lib = L.load()
        n = lib.mla_packed_weights_bytes(C.byref(self.cfg))
        if n == 0:
            raise L.MoEError("mla_packed_weights_bytes", L.MOE_ERR_INVALID_ARG,
                             lib.moe_last_error().decode())
        self.packed = torch.empty(n, dtype=torch.uint8, device=self.device)
        w = L.mla_weights()
        for name in ("w_qa", "s_qa", "w_qb", "s_qb", "w_kva", "s_kva", "w_kvb", "s_kvb", "w_o",
                     "s_o"):
            setattr(w, name, inputs.w[name].data_ptr())
        w.g_qa = inputs.g_qa.data_ptr()
        w.g_kva = inputs.g_kva.data_ptr()
        L.call("mla_pack_weights", C.byref(self.cfg), C.byref(w), self.packed.data_ptr(),
               _stream())
        self._ws = {}

    def workspace(self, n_seq: int, n_new: int, max_len: int) -> torch.Tensor:
        key = (n_seq, n_new, max_len)
        if key not in self._ws:
            n = C.c_size_t(0)
            L.call("mla_workspace_bytes", C.byref(self.cfg), n_seq, n_new, max_len, C.byref(n))
            self._ws[key] = torch.empty(max(n.value, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def forward(self, x, cached_len, cache, n_seq: int, n_new: int, out=None, out_f32=False):
        """out [T, d] bf16 = x + W_o MLA(RMSNorm(x)) (out_f32: fp32 W_o MLA(...)
        without the residual); cache = (codes, scales, rope) of capacity
        cache[0].shape[1]; the new positions are written into it."""
        codes, scales, rope = cache
        max_len = codes.shape[1]
        if out is None:
            out = torch.empty(x.shape, dtype=torch.float32 if out_f32 else x.dtype,
                              device=self.device)
        ws = self.workspace(n_seq, n_new, max_len)
        L.call("mla_forward", C.byref(self.cfg), n_seq, n_new, max_len, _p(x), _p(self.norm_w),
               _p(self.packed), _p(cached_len), _p(codes), _p(scales), _p(rope), _p(out),
               1 if out_f32 else 0, _p(ws), ws.numel(), _stream())
        return out

    def capture_forward(self, x, cached_len, cache, n_seq: int, n_new: int, out):
        """Record mla_forward into a HIP graph (replay with .replay()).

        The workspace is allocated before capture; mla_forward enqueues kernels
        only (no allocation, memset or synchronisation), so the graph replays
        the same launches with the same buffers.  A replay writes the new
        tokens' cache entries again at the same positions.
        """
        self.workspace(n_seq, n_new, cache[0].shape[1])
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):            # one eager call off the default stream
            self.forward(x, cached_len, cache, n_seq, n_new, out=out)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, cached_len, cache, n_seq, n_new, out=out)
        return g

    def attention(self, x, cached_len, cache, n_seq: int, n_new: int):
        """The attention output of every head before W_o: [T, heads * v_head] fp32."""
        codes, scales, rope = cache
        max_len = codes.shape[1]
        T = x.shape[0]
        attn = torch.empty((T, self.shape.n_heads * self.shape.v_head), dtype=torch.float32,
                           device=self.device)
        ws = self.workspace(n_seq, n_new, max_len)
        L.call("mla_attention", C.byref(self.cfg), n_seq, n_new, max_len, _p(x),
               _p(self.norm_w), _p(self.packed), _p(cached_len), _p(codes), _p(scales), _p(rope),
               _p(attn), _p(ws), ws.numel(), _stream())
        return attn
