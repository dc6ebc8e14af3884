/*
 * k2train.h -- C ABI of one training step of the Kimi K2 MoE layer (forward
 * with stored activations, then backward) for AMD Instinct MI355X (gfx950).
 *
 * The layer is the FFN half of a block, out = x + MoE(RMSNorm(x)), as in
 * k2moe.h, trained in BF16 ("Kimi-K2-Base", Pretraining recipe, Training
 * precision): no FP8 in computation, while the inputs of the MoE
 * up-projections and of SwiGLU are kept for the backward as FP8-E4M3 in 1x128
 * tiles with FP32 scales.  Here:
 *   - h = RMSNorm(x) (bf16; the input of the gate/up projections and of the
 *     router) is kept as 1x128 codes hq, hs;
 *   - g, u (each row's gate and up outputs, SwiGLU's inputs, fp32 sums) are
 *     kept as 1x128 codes along the hidden dimension;
 *   - every GEMM is bf16 x bf16 with fp32 accumulation; the backward
 *     recomputes a = silu(g) u from the kept copies, rounds the operands of
 *     its GEMMs (a, w * dy, dg, du, the dequantised h) to bf16, and reads the
 *     kept h for every weight gradient that needs it;
 *   - the top-k choice passes no gradient; the renormalised weights
 *     w = c s_e / sum_j s_j pass theirs to the sigmoid scores and the router;
 *     the correction bias gets none; the bf16 rounding of h passes gradients
 *     straight through.
 *
 * Weights (bf16, caller-owned device memory), "canonical" layout: expert g
 * (g < n_experts routed, then the shared one) at g * 3 * d_ff * d_model
 * elements: gate [d_ff, d_model], up [d_ff, d_model], down [d_model, d_ff]
 * (nn.Linear [out, in]).  The dgrad products read transposed copies made by
 * moe_train_transpose_weights (after every update of the weights).
 * Gradients use the same layout in fp32.
 *
 * Conventions as in k2moe.h (device pointers, row-major, 16-byte aligned
 * unless noted, host validation before any HIP call, enqueue on `stream`,
 * T = 0 enqueues nothing).  Supported: fmt = MOE_FMT_BF16_FP8B128 (bf16
 * activations), dense = 0, d_model % 256 == 0, d_ff % 256 == 0; otherwise
 * MOE_ERR_UNSUPPORTED.  Sums are computed in a fixed order (no floating-point
 * atomics): results are deterministic.
 */
#ifndef K2TRAIN_H
#define K2TRAIN_H

#include <stddef.h>
#include <stdint.h>

#include "k2moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the canonical bf16 expert weights (and of their fp32 gradients:
 * twice this) for n_experts + n_shared experts. */
size_t moe_train_weights_bytes(const moe_config* cfg);

/* Bytes of the transposed copies: per expert down^T [d_ff, d_model] and
 * [gate; up]^T [d_model, 2 d_ff] (bf16), each stored in 32-column K blocks:
 * element (row, k) of a [rows, K] copy at ((k / 32) * rows + row) * 32 + k % 32. */
size_t moe_train_transposed_bytes(const moe_config* cfg);

/* wt <- the transposed copies of w (both canonical / transposed layouts above). */
moe_status moe_train_transpose_weights(const moe_config* cfg, const void* w, void* wt,
                                       void* stream);

/* Bytes of the state the forward keeps for the backward for T tokens:
 * hq [T, d] e4m3, hs [T, d/128] fp32, topk ids [T, k] int32, weights [T, k]
 * fp32, the chosen sigmoid scores [T, k] fp32, the permutation (offsets
 * [n_experts + 1], row_pair [T k], pair_row [T k] int32, as moe_permute), and
 * guq [R, 2 d_ff] e4m3 (g in the first d_ff columns, u in the rest), gus
 * [R, 2 d_ff / 128] fp32, R = T k + T n_shared rows in permuted order (routed
 * rows by expert, then the shared expert's rows by token); each part 256-byte
 * aligned, in that order. */
moe_status moe_train_saved_bytes(const moe_config* cfg, int64_t T, size_t* bytes);

/* Workspace bytes of moe_train_forward and moe_train_backward for T tokens. */
moe_status moe_train_workspace_bytes(const moe_config* cfg, int64_t T, size_t* bytes);

/* Forward of the training step: out [T, d] bf16 = x + MoE(RMSNorm(x)) with
 * bf16 weights w (canonical) and w_router [n_experts, d] bf16, bias fp32
 * (selection only), norm_w bf16; saved receives the state above. */
moe_status moe_train_forward(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                             const void* w_router, const float* bias, const void* w, void* out,
                             void* saved, void* ws, size_t ws_bytes, void* stream);

/* Backward of the training step for the output gradient dout [T, d] bf16,
 * with the same x, norm_w, w_router and w as the forward, the transposed
 * copies wt and the forward's saved state.  Writes (fp32, overwriting):
 *   dx [T, d]; d_norm_w [d]; d_w_router [n_experts, d]; d_w (canonical
 *   layout: every expert's dW_gate, dW_up, dW_down, zeros for experts no
 *   token chose);
 *   optional (NULL to skip): dh_rows [R, d] (each row's dgrad through its
 *   expert before the per-token sum, permuted order) and dw [T, k] (the
 *   gradient of each routing weight). */
/* Streams: the weight-gradient chain runs on a second stream that the
 * library keeps per device (default priority), forked from `stream` after
 * the down dgrad and joined back into it before the call returns, so all of
 * the call's work is ordered after earlier and before later work on `stream`
 * (also under graph capture).  Overlapping calls on one device from several
 * host threads share that stream's events: the caller serializes them. */
moe_status moe_train_backward(const moe_config* cfg, int64_t T, const void* dout, const void* x,
                              const void* norm_w, const void* w_router, const void* w,
                              const void* wt, const void* saved, float* dx, float* d_norm_w,
                              float* d_w_router, float* d_w, float* dh_rows, float* dw, void* ws,
                              size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* K2TRAIN_H */
