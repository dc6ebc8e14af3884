"""Benchmark of the Kimi K2 MoE feed-forward layer on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode|prefill|skewed|dense|ep8_shard]

One step = one moe_forward over one batch: RMSNorm + activation
quantisation, router, top-k, permutation, grouped gate/up GEMM + SwiGLU +
requantisation, grouped down GEMM, combine + residual.  Inputs are seeded
synthetic tensors already resident in HBM; weights are random-init FP8 with
128x128 block scales at the released K2 shape.

Prints one JSON line: tokens/s for the named workload (default: the 64-token
decode step, its timed steps replayed from a HIP graph of moe_forward; --eager
times plain launches), the dominant kernel's roofline fraction measured with
HIP events inside an eager timed region, the whole layer's compulsory bytes
over the step time, the same for the 8192-token prefill, the 16384-token
skewed-routing step and the 4096-token dense FFN, the MLA attention
sub-layer at decode (64 sequences over 4,096 cached positions) and prefill
(2 x 4,096 tokens) with its attention kernel against its roofline, the
shader clock the driver reports while decode and prefill run (sampled from
sysfs after the timed steps), and the CPU oracle timed on the whole decode
batch.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at K2 shape (64-tok decode, 8K prefill); % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# HBM bytes per launch of the gate/up GEMM, from rocprofv3 --pmc FETCH_SIZE (x2.000,
# the factor a 1 GiB copy probe gives) + WRITE_SIZE (x1.000), see
# profiles/gemm_gateup_k2_decode.md; valid only for the GEMM sources whose combined
# sha256 starts with the recorded prefix (null otherwise).
MEASURED_TRAFFIC = {"k2_decode": ("7abebc1c55f983c1", 7.893e9),
                    "k2_prefill": ("7abebc1c55f983c1", 15.166e9)}
# FP8 MFMA busy fraction of the gate/up launch (SQ_VALU_MFMA_BUSY_CYCLES over
# GRBM_GUI_ACTIVE x SIMDs) and its executed/algorithmic MFMA work
# (SQ_INSTS_VALU_MFMA_MOPS_F8 x 512), from rocprofv3 counters, see
# profiles/gemm_mfma_k2_prefill_dense.md; same source-hash rule as the traffic.
MEASURED_MFMA = {"k2_prefill": ("7abebc1c55f983c1", 0.338, 1.041),
                 "k2_dense": ("7abebc1c55f983c1", 0.438, 1.000)}
GEMM_SRCS = [os.path.join(ROOT, "sparse_moe_transformer_sigmoid_amd", "csrc", f)
             for f in ("gemm_fp8_kernel.h", "gemm_fp8.hip", "gemm_fp8_wide.hip")]


def _sources_match(prefix: str) -> bool:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest().startswith(prefix)


def measured_traffic(workload: str):
    rec = MEASURED_TRAFFIC.get(workload)
    return rec[1] if rec is not None and _sources_match(rec[0]) else None


def measured_mfma(workload: str):
    """(MFMA busy fraction, executed / algorithmic MFMA work) or None."""
    rec = MEASURED_MFMA.get(workload)
    return {"mfma_busy": rec[1], "executed_over_algorithmic": rec[2]} \
        if rec is not None and _sources_match(rec[0]) else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skewed", "dense", "ep8_shard"])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the prefill, skewed-routing and dense-FFN lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-step line")
    ap.add_argument("--no-balance", action="store_true",
                    help="skip the routing bias update line")
    ap.add_argument("--no-mla", action="store_true",
                    help="skip the MLA attention decode and prefill lines")
    ap.add_argument("--eager", action="store_true",
                    help="time decode with eager launches instead of a HIP graph")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens of the decode batch the CPU oracle is timed on")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sample (sysfs) after the timed steps")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="also run a plain fp32 copy of BYTES (counter calibration)")
    return ap.parse_args()


def shapes():
    import synth
    return {"decode": synth.K2_DECODE, "prefill": synth.K2_PREFILL,
            "skewed": synth.K2_SKEWED, "dense": synth.K2_DENSE,
            "ep8_shard": synth.K2_EP8_SHARD}


def timed(layer, x, steps, warmup):
    """Run warmup + steps forwards; per-stage HIP-event times of the timed steps."""
    import torch
    from sparse_moe_transformer_sigmoid_amd import _lib as L

    lib = L.load()
    out = torch.empty((x.shape[0], layer.shape.d_model), dtype=x.dtype, device=x.device)
    for _ in range(warmup):
        layer.forward(x, out)
    torch.cuda.synchronize()
    ms = (C.c_double * len(L.STAGES))()
    n = (C.c_int64 * len(L.STAGES))()
    L.check("moe_profile_read", lib.moe_profile_read(ms, n, 1))
    L.check("moe_profile_enable", lib.moe_profile_enable(1))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        layer.forward(x, out)
    stop.record()
    torch.cuda.synchronize()
    L.check("moe_profile_enable", lib.moe_profile_enable(0))
    L.check("moe_profile_read", lib.moe_profile_read(ms, n, 1))
    stage = {name: (ms[i] / n[i] if n[i] else 0.0) for i, name in enumerate(L.STAGES)}
    return start.elapsed_time(stop) / steps, stage


def timed_graph(layer, x, steps, warmup):
    """ms per forward when moe_forward is replayed from a HIP graph."""
    import torch
    out = torch.empty((x.shape[0], layer.shape.d_model), dtype=x.dtype, device=x.device)
    g = layer.capture_forward(x, out)
    for _ in range(warmup):
        g.replay()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(stop) / steps


def routing_stats(layer, x):
    import numpy as np
    import torch
    r = layer.router(x)
    pm = layer.permute(r.ids)
    torch.cuda.synchronize()
    counts = np.diff(pm.offsets.cpu().numpy())
    return int(np.sum(counts > 0)), counts


def layer_bytes(shape, T, touched_all):
    """Compulsory HBM bytes of one forward: the FP8 codes and scales of every
    touched expert (the shared one included), the bf16 router and the fp32
    bias, gamma, x read once and out written once."""
    d, I = shape.d_model, shape.d_ff
    expert = 3 * I * d + 3 * (I // 128) * (d // 128) * 4
    router = 0 if shape.dense else shape.n_experts * d * 2 + shape.n_experts * 4
    return touched_all * expert + router + d * 2 + 2 * T * d * 2


def run_workload(layer, inp, steps, warmup, graph=False):
    shape = inp.shape
    T = inp.x.shape[0]
    layer.use_router(inp)
    ms, stage = timed(layer, inp.x, steps, warmup)
    eager_ms = ms
    if graph:
        ms = timed_graph(layer, inp.x, steps, warmup)
    touched, counts = routing_stats(layer, inp.x)
    touched_all = touched + shape.n_shared
    d, I, k = shape.d_model, shape.d_ff, shape.top_k
    P = T * k
    rows = P + (T if shape.n_shared else 0)
    # gate/up kernel: expert weights read once, activations read once, a_q written once
    gu_bytes = (touched_all * (2 * I * d + 2 * (I // 128) * (d // 128) * 4)
                + T * d + T * (d // 128) * 4 + rows * I + rows * (I // 128) * 4)
    gu_flops = 2.0 * rows * (2 * I) * d
    dn_flops = 2.0 * rows * I * d
    gu_s = stage["gateup"] * 1e-3
    lb = layer_bytes(shape, T, touched_all)
    return dict(T=T, ms=ms, eager_ms=eager_ms, stage=stage, touched=touched_all, counts=counts,
                gu_bytes=gu_bytes, gu_flops=gu_flops, total_flops=gu_flops + dn_flops,
                layer_bytes=lb, layer_gbs=lb / (ms * 1e-3) / 1e9,
                gu_gbs=gu_bytes / gu_s / 1e9 if gu_s > 0 else 0.0,
                gu_tflops=gu_flops / gu_s / 1e12 if gu_s > 0 else 0.0)


def secondary_line(r, workload, sclk=None):
    """Summary of one more workload's run (prefill, skewed routing, dense FFN)."""
    tfl = r["total_flops"] / (r["ms"] * 1e-3) / 1e12
    return {
        "workload": workload, "tokens": r["T"], "value": r["T"] / (r["ms"] * 1e-3),
        "unit": "tokens/s", "ms_per_step": r["ms"], "touched_experts": r["touched"],
        "fp8_tflops_layer": tfl, "frac_fp8_peak_layer": tfl / FP8_PEAK_TFLOPS,
        "layer_bytes": r["layer_bytes"], "layer_gbs": r["layer_gbs"],
        "layer_frac_hbm": r["layer_gbs"] / HBM_PEAK_GBS,
        "gateup_ms": r["stage"]["gateup"],
        "gateup_tflops": r["gu_tflops"], "gateup_frac_fp8_peak": r["gu_tflops"] / FP8_PEAK_TFLOPS,
        "gateup_gbs": r["gu_gbs"], "gateup_frac_hbm_peak": r["gu_gbs"] / HBM_PEAK_GBS,
        "gateup_arithmetic_intensity": r["gu_flops"] / r["gu_bytes"],
        "gateup_traffic": measured_traffic(workload),
        "gateup_mfma_counters": measured_mfma(workload),
        "sclk_mhz": sclk,
        # the published FP8 peak assumes 2400 MHz; at the measured clock:
        "gateup_frac_fp8_peak_at_sclk":
            r["gu_tflops"] / (FP8_PEAK_TFLOPS * sclk / 2400.0) if sclk else None,
        "stage_ms": r["stage"]}


def mla_line(shape, steps, warmup):
    """One MLA attention workload: whole sub-layer time (HIP events on the
    launch stream; decode replayed from a HIP graph, the eager time beside
    it), per-stage times, and the attention stage against its roofline.
    Decode (absorbed form) is bound by HBM: per step it must read every
    attended cache position (656 B: 512 latent codes, 4 scales, 64 bf16
    rotary features) and the absorbed queries and write the latent outputs.
    Prompt-sized batches (>= 128 new tokens per sequence) run the per-head
    form, bound by the bf16 MFMA: 2 (192 + 128) flops per (query, head,
    visible position) plus 2 x 256 x 512 per (position, head) to form the keys
    and values."""
    import numpy as np
    import torch

    import synth
    from sparse_moe_transformer_sigmoid_amd import _lib as L
    from sparse_moe_transformer_sigmoid_amd.mla import K2MLA

    lib = L.load()
    inp = synth.generate_mla(shape, seed=0, device="cuda")
    layer = K2MLA(inp)
    cache = inp.fresh_cache()
    out = torch.empty_like(inp.x)
    S, n = shape.n_seq, shape.n_new
    for _ in range(warmup):
        layer.forward(inp.x, inp.cached_len, cache, S, n, out=out)
    torch.cuda.synchronize()
    nst = len(L.STAGES)
    ms_a, n_a = (C.c_double * nst)(), (C.c_int64 * nst)()
    L.check("moe_profile_read", lib.moe_profile_read(ms_a, n_a, 1))
    L.check("moe_profile_enable", lib.moe_profile_enable(1))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        layer.forward(inp.x, inp.cached_len, cache, S, n, out=out)
    stop.record()
    torch.cuda.synchronize()
    L.check("moe_profile_enable", lib.moe_profile_enable(0))
    L.check("moe_profile_read", lib.moe_profile_read(ms_a, n_a, 1))
    step_ms = start.elapsed_time(stop) / steps
    stage = {nm: ms_a[i] / steps for i, nm in enumerate(L.STAGES) if nm.startswith("mla_")}
    eager_ms = step_ms
    launch = "eager"
    if n == 1:
        # decode: the step replayed from a HIP graph of mla_forward (the same
        # kernels and buffers; per-stage times above are from the eager calls)
        g = layer.capture_forward(inp.x, inp.cached_len, cache, S, n, out)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        step_ms = start.elapsed_time(stop) / steps
        launch = "hip_graph"
        del g
    T, H = shape.tokens, shape.n_heads
    cached = np.asarray(shape.cached, dtype=np.int64)
    visible = int(sum(int(c) * n + n * (n + 1) // 2 for c in cached))   # (query, position) pairs
    attended = int(np.sum(cached + n))                                  # cache rows per sequence
    row_bytes = shape.kv_lora + 4 * (shape.kv_lora // 128) + 2 * shape.qk_rope
    attn_bytes = attended * row_bytes + T * H * (shape.kv_lora + shape.qk_rope) * 4 + \
        T * H * shape.kv_lora * 4
    per_head = n >= 128
    if per_head:
        dqk, dv = shape.qk_nope + shape.qk_rope, shape.v_head
        attn_flops = 2.0 * visible * H * (dqk + dv) + \
            2.0 * attended * H * (shape.qk_nope + shape.v_head) * shape.kv_lora
        # each fp32 operand enters the bf16 MFMA as high and low halves: three
        # products per key/value feature, two per rotary one
        mfma_flops = 2.0 * visible * H * (3 * shape.qk_nope + 2 * shape.qk_rope + 3 * dv) + \
            2.0 * attended * H * (shape.qk_nope + shape.v_head) * shape.kv_lora
        # cache rows in; keys and values (two bf16 halves) written and read back
        # once; queries in, output codes out
        attn_bytes = attended * row_bytes + \
            2 * attended * H * (shape.qk_nope + shape.v_head) * 4 + T * H * (dqk * 4 + shape.v_head)
        kern = "mla_kv_expand_kernel + mla_mha_kernel"
    else:
        attn_flops = 2.0 * visible * H * ((shape.kv_lora + shape.qk_rope) + shape.kv_lora)
        mfma_flops = 2.0 * attn_flops
        kern = "mla_attn_kernel"
    a_ms = stage["mla_attn"]
    w_bytes = sum(v.numel() * v.element_size() for v in inp.w.values())
    layer_bytes = w_bytes + attended * row_bytes + 2 * T * shape.d_model * 2
    line = {"workload": shape.name, "sequences": S, "new_tokens_per_sequence": n,
            "cached_per_sequence": sorted(set(int(c) for c in cached)), "tokens": T,
            "ms_per_step": step_ms, "eager_ms_per_step": eager_ms, "launch": launch,
            "value": T / (step_ms * 1e-3), "unit": "tokens/s",
            "form": "per-head" if per_head else "absorbed",
            "stage_ms": stage, "layer_bytes": layer_bytes,
            "layer_frac_hbm": layer_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    ai = attn_flops / attn_bytes
    if ai < BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS:
        gbs = attn_bytes / (a_ms * 1e-3) / 1e9
        line["roofline"] = {"kernel": kern, "bound": "hbm", "achieved": gbs,
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                            "kernel_ms": a_ms, "algorithmic_bytes": attn_bytes,
                            "algorithmic_flops": attn_flops, "arithmetic_intensity": ai}
    else:
        tf = attn_flops / (a_ms * 1e-3) / 1e12
        line["roofline"] = {"kernel": kern, "bound": "mfma", "achieved": tf,
                            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": tf / BF16_PEAK_TFLOPS, "kernel_ms": a_ms,
                            "algorithmic_bytes": attn_bytes, "algorithmic_flops": attn_flops,
                            "arithmetic_intensity": ai,
                            "executed_mfma_tflops": mfma_flops / (a_ms * 1e-3) / 1e12,
                            "note": "bf16 MFMA peak; fp32 operands enter the MFMA as high "
                                    "and low bf16 halves, so the executed MFMA work "
                                    "(executed_mfma_tflops) exceeds the algorithmic flops"}
    del layer, inp, cache
    return line


def balance_line(steps, warmup):
    """One training step's routing bias update at the K2 prefill batch: zero
    the loads, count the 8,192 x 8 top-k choices over 384 experts
    (moe_expert_load), update the bias (moe_bias_update).  Algorithmic bytes:
    the choices read once, the loads written and read back, the bias read and
    written.  The step is a handful of small launches, so its time is launch
    latency rather than bandwidth; it runs once per training step."""
    import torch

    import synth
    from sparse_moe_transformer_sigmoid_amd import _lib as L
    from sparse_moe_transformer_sigmoid_amd.layer import config_from_shape

    shape = synth.K2_PREFILL
    E, k, T = shape.n_experts, shape.top_k, shape.tokens
    cfg = config_from_shape(shape)
    ids = synth.topk_choices(T, k, E, seed=0, skew=0.5, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    bias = synth.bias_values(E, seed=0, device="cuda")
    s = torch.cuda.current_stream()
    sp = C.c_void_p(s.cuda_stream)

    def one():
        counts.zero_()
        L.call("moe_expert_load", C.byref(cfg), T, ids.data_ptr(), counts.data_ptr(), sp)
        L.call("moe_bias_update", C.byref(cfg), counts.data_ptr(), C.c_float(1e-3),
               bias.data_ptr(), sp)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(steps):
        one()
    stop.record(s)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = T * k * 4 + 2 * E * 4 + 2 * E * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "bias_update_k2_prefill", "choices": T * k, "experts": E,
            "ms_per_step": ms, "algorithmic_bytes": nbytes,
            "roofline": {"kernel": "expert_load_kernel + bias_update_kernel", "bound": "hbm",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "note": "three small launches (zero, count, update): latency-bound"}}


def train_line(steps, warmup):
    """One training step of the MoE layer at the K2 prefill batch (8,192
    tokens, 384 + 1 experts, bf16 weights): moe_train_forward (keeping FP8
    copies) then moe_train_backward (all gradients), HIP events on the launch
    stream, per-stage times from the library's profiler.  Algorithmic work:
    18 R I d bf16 flops (R = T k + T rows; forward 6 R I d, dgrad 6 R I d,
    wgrad 6 R I d) and, as bytes, the weights read (bf16, twice: forward and
    transposed copies for dgrad) plus the fp32 weight gradients written."""
    import torch

    import synth
    from sparse_moe_transformer_sigmoid_amd import _lib as L
    from sparse_moe_transformer_sigmoid_amd.train import K2Train

    lib = L.load()
    sh = synth.K2_PREFILL
    inp = synth.generate_train(sh, seed=0, device="cuda")
    layer = K2Train(inp)
    T, d, I = sh.tokens, sh.d_model, sh.d_ff
    G = sh.n_experts + sh.n_shared
    out = torch.empty_like(inp.x)
    saved = layer.saved_buffer(T)
    grads = None

    def one():
        nonlocal grads
        layer.forward(inp.x, saved, out)
        grads = layer.backward(inp.dout, inp.x, saved, grads)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    nst = len(L.STAGES)
    ms_a, n_a = (C.c_double * nst)(), (C.c_int64 * nst)()
    L.check("moe_profile_read", lib.moe_profile_read(ms_a, n_a, 1))
    L.check("moe_profile_enable", lib.moe_profile_enable(1))
    s = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(steps):
        one()
    stop.record(s)
    torch.cuda.synchronize()
    L.check("moe_profile_enable", lib.moe_profile_enable(0))
    L.check("moe_profile_read", lib.moe_profile_read(ms_a, n_a, 1))
    ms = start.elapsed_time(stop) / steps
    stage = {nm: ms_a[i] / steps for i, nm in enumerate(L.STAGES) if ms_a[i] > 0}
    # the dgrad products read transposed copies of the weights, which must be
    # refreshed (moe_train_transpose_weights) after every weight update: once
    # per optimizer step, outside the forward + backward timed above
    start.record(s)
    for _ in range(3):
        layer.transpose_weights()
    stop.record(s)
    torch.cuda.synchronize()
    copy_ms = start.elapsed_time(stop) / 3
    R = T * sh.top_k + T * sh.n_shared
    flops = 18.0 * R * I * d
    nbytes = 2 * G * 3 * I * d * 2 + G * 3 * I * d * 4
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {"workload": "k2_prefill_train_step", "tokens": T, "rows": R, "ms_per_step": ms,
            "value": T / (ms * 1e-3), "unit": "tokens/s", "stage_ms": stage,
            "weight_copy_ms": copy_ms, "ms_per_step_with_weight_copy": ms + copy_ms,
            "algorithmic_tflop": flops / 1e12, "bf16_tflops": tf,
            "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            # 18 R I d flops over the bytes below is ~144 flop/B, under the bf16
            # ridge point (312 flop/B): the step's roofline is HBM
            "roofline": {"kernel": "whole step", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "algorithmic_bytes": nbytes,
                         "note": "bf16 expert weights read twice (forward; transposed copies "
                                 "for dgrad) and fp32 weight gradients written once"}}
    del layer, inp, grads, saved, out
    torch.cuda.empty_cache()
    return line


def sclk_file():
    """The amdgpu driver's shader-clock table of the GPU torch uses (sysfs
    pp_dpm_sclk, found by the device's PCI address), or None."""
    import torch
    p = torch.cuda.get_device_properties(torch.cuda.current_device())
    path = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
            f"{p.pci_device_id:02x}.0/pp_dpm_sclk")
    return path if os.path.exists(path) else None


def sclk_during(layer, x, seconds=1.5):
    """Median shader clock (MHz) while the step runs back to back, outside the
    timed region: the level the driver marks current in pp_dpm_sclk, read
    from sysfs every 50 ms (no child process).  None if the file is absent.
    The FP8 and bf16 peaks assume 2.4 GHz, which sustained MFMA work does
    not hold."""
    import re
    import statistics
    import threading

    import torch
    path = sclk_file()
    if path is None:
        return None
    vals, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                with open(path) as f:
                    for line in f:
                        m = re.search(r"(\d+)\s*Mhz\s*\*", line, re.IGNORECASE)
                        if m:
                            vals.append(int(m.group(1)))
            except OSError:
                return
            stop.wait(0.05)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.time()
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(10):
            layer.forward(x)
        torch.cuda.synchronize()
    stop.set()
    th.join()
    vals = vals[2:] if len(vals) > 4 else vals     # the first may precede the load
    return int(statistics.median(vals)) if vals else None


def cpu_baseline(inp, n_tokens, runs=3):
    """The oracle on the host cores, end to end on the first n_tokens of the
    batch (routing of the batch, every expert those tokens use): median of
    `runs` runs, one run if the first takes over 60 s."""
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.adapt import to_f32
    from oracle.moe_ref import moe_layer, params_from_shape, rmsnorm, route

    p = params_from_shape(inp.shape)
    T = inp.x.shape[0]
    sel = np.arange(min(n_tokens, T))
    x = to_f32(inp.x)
    norm_w = to_f32(inp.norm_w)
    wr = None if inp.w_router is None else to_f32(inp.w_router)
    bias = None if inp.bias is None else to_f32(inp.bias)
    # host copies of every expert the sample needs (the FP8 codes and scales as
    # they sit in memory), made before the clock starts
    h = rmsnorm(x[sel], norm_w, p.rms_eps, round_bf16=p.fp8)
    need = set(range(p.n_experts, p.n_experts + p.n_shared))
    if p.dense:
        need.add(0)
    else:
        need.update(np.unique(route(h, wr, bias, p.top_k, p.routed_scaling,
                                    p.norm_topk_prob)["ids"]).tolist())
    cache = {}
    for e in need:
        cache[e] = {n: (None if getattr(inp, n) is None else getattr(inp, n)[e].cpu().numpy())
                    for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        moe_layer(p, x, norm_w, wr, bias, lambda e: cache[e], tokens=sel)
        times.append(time.perf_counter() - t0)
        if times[0] > 60.0:
            break
    dt = statistics.median(times)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    whole = len(sel) == T
    what = (f"the whole {T}-token {inp.shape.name} batch" if whole else
            f"the first {len(sel)} of {T} tokens of the {inp.shape.name} batch")
    return {"value": len(sel) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}: routing, every touched expert dequantised and applied, combine; "
                      f"median of {len(times)} run(s) ({', '.join(f'{t:.1f}' for t in times)} s) "
                      f"on {os.cpu_count()} host cores, BLAS threads {threads}",
            "experts_touched": len(need)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not "
                                   "supported (the layer is not sharded across GPUs)"}))
        sys.exit(2)
    import torch

    import synth
    from sparse_moe_transformer_sigmoid_amd.layer import K2MoE

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    shp = shapes()[args.workload]
    t0 = time.time()
    if args.workload in ("dense", "ep8_shard"):
        base = synth.generate(shp, seed=0, device="cuda")
        inp = base
    else:
        base = synth.generate(synth.K2_DECODE, seed=0, device="cuda")
        inp = synth.with_workload(base, shp, seed=0)
    layer = K2MoE(base)
    print(f"# inputs generated and packed in {time.time() - t0:.1f} s", file=sys.stderr,
          flush=True)

    # decode is launch-sensitive: the timed steps replay moe_forward from a HIP
    # graph (the same kernels and buffers); the eager time is reported beside it
    graph = args.workload == "decode" and not args.eager
    res = run_workload(layer, inp, args.steps, args.warmup, graph=graph)
    T = res["T"]
    value = T / (res["ms"] * 1e-3)
    gu_ms = res["stage"]["gateup"]
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms"],
        "eager_ms_per_step": res["eager_ms"], "launch": "hip_graph" if graph else "eager",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": shp.name, "tokens": T, "d_model": shp.d_model,
                   "routed_experts": shp.n_experts, "shared_experts": shp.n_shared,
                   "top_k": shp.top_k, "d_ff": shp.d_ff,
                   "touched_experts": res["touched"]},
        "roofline": {"bound": "hbm", "kernel": "grouped gate/up GEMM + SwiGLU + requant",
                     "achieved": res["gu_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": res["gu_gbs"] / HBM_PEAK_GBS,
                     "traffic": measured_traffic(shp.name),
                     "mfma_counters": measured_mfma(shp.name),
                     "kernel_ms": gu_ms, "algorithmic_bytes": res["gu_bytes"]},
        "stage_ms": res["stage"],
    }
    # the kernel's bound follows its arithmetic intensity: below the ridge point
    # (peak flops / peak bandwidth) HBM bounds it, above it the FP8 MFMA peak
    ai = res["gu_flops"] / res["gu_bytes"]
    attainable_tflops = min(FP8_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    line["roofline"].update({"arithmetic_intensity": ai, "algorithmic_flops": res["gu_flops"],
                             "fp8_tflops": res["gu_tflops"],
                             "frac_fp8_peak": res["gu_tflops"] / FP8_PEAK_TFLOPS,
                             "frac_attainable": res["gu_tflops"] / attainable_tflops})
    if ai > FP8_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS:
        line["roofline"].update({"bound": "mfma", "achieved": res["gu_tflops"],
                                 "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": res["gu_tflops"] / FP8_PEAK_TFLOPS})
    line["layer"] = {"bytes": res["layer_bytes"], "gbs": res["layer_gbs"],
                     "frac_hbm": res["layer_gbs"] / HBM_PEAK_GBS,
                     "note": "compulsory bytes of the whole forward (touched experts' FP8 "
                             "codes and scales, router, bias, gamma, x read and out written "
                             "once) over ms_per_step"}
    if args.workload == "decode" and not args.no_secondary:
        sub = max(3, args.steps // 2)
        pre = synth.with_workload(base, synth.K2_PREFILL, seed=0)
        rp = run_workload(layer, pre, sub, 2)
        sclk = None if args.no_clock else sclk_during(layer, pre.x)
        line["prefill"] = secondary_line(rp, pre.shape.name, sclk)
        print(f"# prefill {rp['ms']:.3f} ms", file=sys.stderr, flush=True)
        del pre
        skw = synth.with_workload(base, synth.K2_SKEWED, seed=0)
        rs = run_workload(layer, skw, sub, 2)
        line["skewed"] = secondary_line(rs, skw.shape.name)
        line["skewed"]["max_rows_per_expert"] = int(rs["counts"].max())
        line["skewed"]["experts_under_10_rows"] = int((rs["counts"] < 10).sum())
        print(f"# skewed {rs['ms']:.3f} ms", file=sys.stderr, flush=True)
        del skw
        dense = synth.generate(synth.K2_DENSE, seed=0, device="cuda")
        dlayer = K2MoE(dense)
        rd = run_workload(dlayer, dense, sub, 2)
        line["dense"] = secondary_line(rd, dense.shape.name)
        print(f"# dense {rd['ms']:.3f} ms", file=sys.stderr, flush=True)
        del dlayer, dense
    if args.workload == "decode" and not args.no_mla:
        line["mla"] = {}
        for nm, shp_m in (("decode", synth.MLA_K2_DECODE), ("prefill", synth.MLA_K2_PREFILL)):
            line["mla"][nm] = mla_line(shp_m, max(3, args.steps // 2), 2)
            print(f"# mla {nm} {line['mla'][nm]['ms_per_step']:.3f} ms", file=sys.stderr,
                  flush=True)
    if args.workload == "decode" and not args.no_train:
        line["train"] = train_line(max(3, args.steps // 4), 2)
        print(f"# training step {line['train']['ms_per_step']:.2f} ms", file=sys.stderr, flush=True)
    if args.workload == "decode" and not args.no_balance:
        line["bias_update"] = balance_line(max(10, args.steps), 3)
        print(f"# bias update {line['bias_update']['ms_per_step'] * 1e3:.1f} us", file=sys.stderr,
              flush=True)
    if not args.no_clock:
        layer.use_router(inp)
        line["sclk_mhz"] = sclk_during(layer, inp.x)
    if args.copy_probe:
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)       # reads and writes copy_probe bytes
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = n * 4
        del src, dst
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens, args.cpu_runs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
