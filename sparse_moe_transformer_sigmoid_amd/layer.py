"""PyTorch-side wrapper: device buffers and streams for the C ABI.

torch allocates the tensors and supplies the stream; each method marshals
pointers into one ABI call.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib as L


def config_from_shape(shape) -> L.moe_config:
    """moe_config for a workload shape (fields named as in config.json)."""
    c = L.moe_config()
    c.d_model = shape.d_model
    c.n_experts = shape.n_experts
    c.n_shared = shape.n_shared
    c.top_k = shape.top_k
    c.d_ff = shape.d_ff
    c.n_group = 1
    c.topk_group = 1
    c.norm_topk_prob = 1 if shape.norm_topk_prob else 0
    c.fmt = L.MOE_FMT_BF16_FP8B128 if shape.fmt == "fp8" else L.MOE_FMT_F32
    c.dense = 1 if shape.dense else 0
    c.routed_scaling = shape.routed_scaling
    c.rms_eps = shape.rms_eps
    return c


def _p(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def workspace_bytes(cfg: L.moe_config, T: int, entry: int) -> int:
    n = C.c_size_t(0)
    L.call("moe_workspace_bytes", C.byref(cfg), T, entry, C.byref(n))
    return n.value


@dataclass
class RouterOut:
    ids: torch.Tensor
    w: torch.Tensor
    gap: torch.Tensor
    xq: torch.Tensor
    xs: torch.Tensor | None


@dataclass
class PermuteOut:
    offsets: torch.Tensor
    row_pair: torch.Tensor
    pair_row: torch.Tensor


class K2MoE:
    """One MoE layer with packed weights resident on the GPU."""

    def __init__(self, inputs, device="cuda"):
        self.shape = inputs.shape
        self.cfg = config_from_shape(self.shape)
        self.device = torch.device(device)
        self.fp8 = self.shape.fmt == "fp8"
        self.w_router = inputs.w_router
        self.bias = inputs.bias
        self.norm_w = inputs.norm_w
        nbytes = L.load().moe_packed_weights_bytes(C.byref(self.cfg))
        if nbytes == 0:
            raise L.MoEError("moe_packed_weights_bytes", L.MOE_ERR_INVALID_ARG,
                             L.load().moe_last_error().decode())
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        NE = self.shape.n_experts + self.shape.n_shared
        arr = (L.moe_expert_w * NE)()
        for e in range(NE):
            arr[e].w_gate = inputs.w_gate[e].data_ptr()
            arr[e].w_up = inputs.w_up[e].data_ptr()
            arr[e].w_down = inputs.w_down[e].data_ptr()
            if self.fp8:
                arr[e].s_gate = inputs.s_gate[e].data_ptr()
                arr[e].s_up = inputs.s_up[e].data_ptr()
                arr[e].s_down = inputs.s_down[e].data_ptr()
        L.call("moe_pack_weights", C.byref(self.cfg), arr, NE, self.packed.data_ptr(), _stream())
        torch.cuda.current_stream().synchronize()
        self._ws = {}

    def use_router(self, inputs) -> "K2MoE":
        """Take the norm weight, router weight and correction bias of ``inputs``
        (workloads of one layer share the experts but may differ in the bias)."""
        self.norm_w = inputs.norm_w
        self.w_router = inputs.w_router
        self.bias = inputs.bias
        return self

    # ------------------------------------------------------------- buffers
    def workspace(self, T: int, entry: int) -> torch.Tensor:
        key = (T, entry)
        if key not in self._ws:
            n = workspace_bytes(self.cfg, T, entry)
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def _act_dtype(self):
        return torch.bfloat16 if self.fp8 else torch.float32

    # ------------------------------------------------------------- entry points
    def router(self, x: torch.Tensor) -> RouterOut:
        T, d, k = x.shape[0], self.shape.d_model, self.shape.top_k
        dev = self.device
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        gap = torch.empty((T,), dtype=torch.float32, device=dev)
        if self.fp8:
            xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            xs = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
        else:
            xq = torch.empty((T, d), dtype=torch.float32, device=dev)
            xs = None
        ws = self.workspace(T, L.MOE_WS_ROUTER)
        L.call("moe_router", C.byref(self.cfg), T, _p(x), _p(self.norm_w), _p(self.w_router),
               _p(self.bias), _p(ids), _p(w), _p(gap), _p(xq), _p(xs), _p(ws), ws.numel(),
               _stream())
        return RouterOut(ids, w, gap, xq, xs)

    def permute(self, ids: torch.Tensor) -> PermuteOut:
        T = ids.shape[0]
        P = ids.numel()
        dev = self.device
        offsets = torch.empty((self.shape.n_experts + 1,), dtype=torch.int32, device=dev)
        row_pair = torch.empty((P,), dtype=torch.int32, device=dev)
        pair_row = torch.empty((P,), dtype=torch.int32, device=dev)
        ws = self.workspace(T, L.MOE_WS_PERMUTE)
        L.call("moe_permute", C.byref(self.cfg), T, _p(ids), _p(offsets), _p(row_pair),
               _p(pair_row), _p(ws), ws.numel(), _stream())
        return PermuteOut(offsets, row_pair, pair_row)

    def grouped_swiglu(self, T: int, xq, xs, offsets, row_pair, return_act: bool = False):
        """Expert rows and shared output; with return_act (FP8 format) also the
        requantised SwiGLU activations (codes [rows, d_ff], scales [rows, d_ff/128])."""
        d, I = self.shape.d_model, self.shape.d_ff
        P = T * self.shape.top_k
        rows = torch.empty((P, d), dtype=torch.float32, device=self.device)
        shared = (torch.empty((T, d), dtype=torch.float32, device=self.device)
                  if self.shape.n_shared else None)
        act_q = act_s = None
        if return_act and self.fp8:
            nrows = P + (T if self.shape.n_shared else 0)
            act_q = torch.empty((nrows, I), dtype=torch.uint8, device=self.device)
            act_s = torch.empty((nrows, I // 128), dtype=torch.float32, device=self.device)
        ws = self.workspace(T, L.MOE_WS_SWIGLU)
        L.call("moe_grouped_swiglu", C.byref(self.cfg), T, _p(xq), _p(xs), _p(offsets),
               _p(row_pair), _p(self.packed), _p(rows), _p(shared), _p(act_q), _p(act_s),
               _p(ws), ws.numel(), _stream())
        if return_act:
            return rows, shared, act_q, act_s
        return rows, shared

    def combine(self, rows, pair_row, w, shared, residual=None, out_f32=False):
        T = pair_row.numel() // self.shape.top_k
        dt = torch.float32 if (out_f32 or not self.fp8) else torch.bfloat16
        out = torch.empty((T, self.shape.d_model), dtype=dt, device=self.device)
        L.call("moe_combine", C.byref(self.cfg), T, _p(rows), _p(pair_row), _p(w), _p(shared),
               _p(residual), _p(out), 1 if out_f32 else 0, _stream())
        return out

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.shape.d_model), dtype=self._act_dtype(), device=self.device)
        ws = self.workspace(T, L.MOE_WS_FORWARD)
        L.call("moe_forward", C.byref(self.cfg), T, _p(x), _p(self.norm_w), _p(self.w_router),
               _p(self.bias), _p(self.packed), _p(out), _p(ws), ws.numel(), _stream())
        return out

    def forward_noalloc(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """moe_forward_noalloc: the library's static scratch array as workspace."""
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.shape.d_model), dtype=self._act_dtype(), device=self.device)
        L.call("moe_forward_noalloc", C.byref(self.cfg), T, _p(x), _p(self.norm_w),
               _p(self.w_router), _p(self.bias), _p(self.packed), _p(out), _stream())
        return out

    def expert_load(self, topk_ids: torch.Tensor,
                    counts: torch.Tensor | None = None) -> torch.Tensor:
        """moe_expert_load: add the expert loads of topk_ids [T, k] int32 into
        counts (int32 [n_experts]; a zeroed one when None)."""
        if counts is None:
            counts = torch.zeros(self.shape.n_experts, dtype=torch.int32, device=self.device)
        L.call("moe_expert_load", C.byref(self.cfg), topk_ids.shape[0], _p(topk_ids),
               _p(counts), _stream())
        return counts

    def bias_update(self, counts: torch.Tensor, speed: float,
                    bias: torch.Tensor | None = None) -> torch.Tensor:
        """moe_bias_update, in place on bias (default: this layer's routing bias)."""
        b = self.bias if bias is None else bias
        L.call("moe_bias_update", C.byref(self.cfg), _p(counts), C.c_float(speed), _p(b),
               _stream())
        return b

    def capture_forward(self, x: torch.Tensor, out: torch.Tensor) -> torch.cuda.CUDAGraph:
        """Record moe_forward(x) -> out into a HIP graph (replay with .replay()).

        The workspace for x's token count is allocated before capture; moe_forward
        enqueues kernels only (no allocation, memset or synchronisation), so the
        graph replays the same launches with the same buffers.
        """
        self.workspace(x.shape[0], L.MOE_WS_FORWARD)
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):            # one eager call off the default stream
            self.forward(x, out)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, out)
        return g
