/*
 * k2moe.h -- C ABI of the Kimi K2 sparse-MoE feed-forward layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer is the FFN half of a Kimi K2 decoder block ("Kimi K2 · Dense
 * transformer block", Code: post-attention RMSNorm, then the MLP, then the
 * residual add):
 *
 *     out = x + MoE(RMSNorm(x))
 *     MoE(h) = sum_{e in top-k(h)} w_e * E_e(h) + E_shared(h)
 *     E(h)   = W_down (silu(W_gate h) * (W_up h))
 *
 * with sigmoid router scores, a correction bias used for the top-k choice
 * only, renormalised weights times the routed scaling factor ("Kimi-K2-Base",
 * Mixture of experts) and FP8 e4m3 weights in 128x128 blocks with
 * dynamically quantised 1x128 activations ("Kimi K2 · Architecture",
 * config.json quantization_config; "Kimi-K2-Base", Pretraining recipe,
 * Training precision).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major.
 *    Buffers the kernels access in vectors (x, norm_w, w_router, xq, rows,
 *    shared_out, residual, out, packed weights, workspace, expert codes) must
 *    be 16-byte aligned; scales, bias, ids, weights, gap and index arrays
 *    4-byte aligned.  Nothing here allocates device memory except through
 *    the caller's workspace, and nothing is kept between calls.  Calls that
 *    may run at the same time (on different streams) need their own
 *    workspaces and outputs; read-only inputs (weights, x) may be shared.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns without synchronising; device faults
 *    surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call; on error
 *    nothing is enqueued and moe_last_error() describes the problem.
 *  - T (tokens) = 0 is valid: tensor pointers are not examined and nothing
 *    is enqueued.  The kernels use 32-bit row offsets: T <= 2^24 and
 *    T * (top_k + 1) * max(d_model, d_ff) < 2^32 (K2: T <= 66,576 per call);
 *    larger T gives MOE_ERR_UNSUPPORTED.
 *  - Results are bitwise deterministic: no floating-point atomics.
 *
 * Formats (moe_config.fmt):
 *  MOE_FMT_BF16_FP8B128: x, norm weight, router weight and out are bf16;
 *    correction bias fp32; expert weights are e4m3 (OCP E4M3FN) codes, one
 *    byte each, in nn.Linear [out, in] layout with one fp32 scale per 128x128
 *    block stored row-major as [out/128, in/128]; activations are quantised
 *    per token and 128 columns: scale = amax/448, code = e4m3(x/scale).
 *  MOE_FMT_F32: everything fp32, no quantisation.
 */
#ifndef K2MOE_H
#define K2MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or shape */
  MOE_ERR_UNSUPPORTED = 2,  /* a configuration the kernels do not implement */
  MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4           /* a HIP launch or copy failed */
} moe_status;

typedef enum { MOE_FMT_F32 = 0, MOE_FMT_BF16_FP8B128 = 1 } moe_fmt;

/* Layer configuration, host memory.  Mirrors the released config.json keys
 * ("Kimi K2 · Architecture", Sources, config.json): hidden_size,
 * n_routed_experts, n_shared_experts, num_experts_per_tok,
 * moe_intermediate_size, n_group, topk_group, norm_topk_prob,
 * routed_scaling_factor, rms_norm_eps.
 *  - n_group and topk_group must be 1 (K2 uses one expert group);
 *  - n_shared is 0 or 1 (K2: 1);
 *  - dense = 1 runs the first block's dense SwiGLU as one expert with
 *    weight routed_scaling and no router: n_experts = top_k = 1, n_shared = 0.
 * FP8 format limits: d_model % 256 == 0, d_model <= 16384, d_ff % 128 == 0,
 * d_ff <= 65536,
 * n_experts % 16 == 0 unless dense.  F32 format: d_model % 8 == 0,
 * d_model <= 16384.  Both: top_k <= 32, n_experts <= 1024. */
typedef struct {
  int32_t d_model;        /* 7168 */
  int32_t n_experts;      /* routed experts, 384 */
  int32_t n_shared;       /* 1 */
  int32_t top_k;          /* 8 */
  int32_t d_ff;           /* hidden features per expert, 2048 (dense: 18432) */
  int32_t n_group;        /* 1 */
  int32_t topk_group;     /* 1 */
  int32_t norm_topk_prob; /* 1: renormalise the selected weights to sum 1 */
  int32_t fmt;            /* moe_fmt */
  int32_t dense;          /* 0, or 1 for the dense FFN */
  float routed_scaling;   /* 2.827 */
  float rms_eps;          /* 1e-6 */
} moe_config;

/* One expert's weights in canonical layout (device pointers).
 * w_gate, w_up: [d_ff, d_model]; w_down: [d_model, d_ff]; e4m3 codes (uint8)
 * or fp32.  s_*: fp32 block scales [rows/128, cols/128]; NULL for F32. */
typedef struct {
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
} moe_expert_w;

/* Status name ("MOE_OK", ...). */
const char* moe_status_str(moe_status s);
/* Detail of the last non-OK status returned on this host thread. */
const char* moe_last_error(void);

/* Size of the packed weight buffer for n_experts + n_shared experts. */
size_t moe_packed_weights_bytes(const moe_config* cfg);

/* One-time re-layout of the expert weights into the packed buffer read by
 * the grouped GEMMs (model-load step, not part of a forward pass).
 * experts: HOST array of n_experts + n_shared descriptors, routed experts
 * first, shared expert last.  packed: device buffer of
 * moe_packed_weights_bytes() bytes.  FP8 layout: per expert, gate and up
 * rows are interleaved per 128 hidden features and cut into 16-row x
 * 128-column MFMA fragments stored in the order one wavefront streams
 * them; scales follow all experts' codes. */
moe_status moe_pack_weights(const moe_config* cfg, const moe_expert_w* experts,
                            int32_t n_experts_total, void* packed, void* stream);

typedef enum {
  MOE_WS_ROUTER = 0,
  MOE_WS_PERMUTE = 1,
  MOE_WS_SWIGLU = 2,
  MOE_WS_FORWARD = 3
} moe_ws_entry;

/* Workspace bytes the named entry point needs for T tokens. */
moe_status moe_workspace_bytes(const moe_config* cfg, int64_t T, int32_t entry,
                               size_t* bytes);

/* RMSNorm, activation quantisation and routing.
 * ("Kimi-K2-Base", Normalization and stability: RMSNorm, eps 1e-6;
 *  Mixture of experts: sigmoid score, correction bias added for the top-k
 *  choice only, one group, renormalised top-k weights times 2.827.)
 *  x [T, d], norm_w [d]: bf16 (FP8 format) or fp32.
 *  w_router [E, d] (bf16 / fp32), bias [E] fp32: may be NULL when dense.
 *  h = RMSNorm(x): mean of squares rounded to fp32, r = 1/sqrt(ms + eps),
 *    h = bf16((x r) gamma) (fp32 format: no rounding).
 *  xq: FP8 format: [T, d] e4m3 codes of h, xs: [T, d/128] fp32 scales;
 *      F32 format: xq is h as fp32 [T, d] and xs must be NULL.
 *  topk_ids [T, k] int32, ascending per token; topk_w [T, k] fp32 in the
 *  same order; gap [T] fp32 (nullable) = k-th minus (k+1)-th biased score
 *  (+inf when k = E or dense).  Top-k ties go to the lower expert id. */
moe_status moe_router(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                      const void* w_router, const float* bias, int32_t* topk_ids,
                      float* topk_w, float* gap, void* xq, float* xs, void* ws,
                      size_t ws_bytes, void* stream);

/* Group the T*k (token, slot) pairs by expert, stable in token order.
 * The gate scores every token of the batch as one flat list of bsz*seq_len
 * rows ("Kimi-K2-Base", Mixture of experts, Load balancing: the scores are
 * viewed as bsz*seq_len rows before the bias is added), and each chosen
 * expert is then applied to the tokens that chose it; this call builds that
 * token-to-expert grouping for the grouped GEMMs.
 *  expert_offsets [E+1]: exclusive prefix sum of the per-expert counts
 *  (expert_offsets[E] = T*k); row_pair [T*k]: pair index t*k+slot of each
 *  permuted row; pair_row [T*k]: its inverse.  Bit-exact, no atomics order.
 *  topk_ids must hold k distinct ids in [0, E) per token (as moe_router
 *  writes them); other values give unspecified results but every access
 *  stays inside the buffers. */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* row_pair, int32_t* pair_row,
                       void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU experts ("Kimi-K2-Base", Feed-forward, Activation:
 * down(silu(gate(x)) * up(x)), no biases).  FP8 format: block-scaled FP8
 * GEMMs with fp32 accumulation; the SwiGLU output is requantised per 1x128
 * before the down projection.
 *  xq, xs: from moe_router.  expert_offsets, row_pair: from moe_permute.
 *  packed_w: from moe_pack_weights.
 *  rows [T*k, d] fp32: unweighted expert output of each permuted row.
 *  shared_out [T, d] fp32: shared expert output; NULL iff n_shared == 0.
 *  act_q, act_s (nullable, FP8 format only, both or neither): where the
 *  requantised SwiGLU activations of the permuted rows go, instead of the
 *  workspace: act_q [T*k + n_shared*T, d_ff] e4m3 codes, act_s [same rows,
 *  d_ff/128] fp32 scales; the shared expert's rows follow the routed ones. */
moe_status moe_grouped_swiglu(const moe_config* cfg, int64_t T, const void* xq,
                              const float* xs, const int32_t* expert_offsets,
                              const int32_t* row_pair, const void* packed_w, float* rows,
                              float* shared_out, void* act_q, float* act_s, void* ws,
                              size_t ws_bytes, void* stream);

/* Weighted combine plus residual ("Kimi K2 · Dense transformer block", Code:
 * residual add after the MLP).  For each token, in ascending expert order:
 *   y = sum_slot topk_w * rows[pair_row[t*k+slot]]  (+ shared_out[t])
 *   out = x + y, rounded once to the output type.
 *  residual: x [T, d] in the layer dtype, or NULL for out = y.
 *  out_f32 = 0: out has the layer dtype (bf16 / fp32); 1: fp32. */
moe_status moe_combine(const moe_config* cfg, int64_t T, const float* rows,
                       const int32_t* pair_row, const float* topk_w, const float* shared_out,
                       const void* residual, void* out, int32_t out_f32, void* stream);

/* The whole layer in one call: out [T, d] (layer dtype) = x + MoE(RMSNorm(x)),
 * the FFN half of a decoder block ("Kimi K2 · Dense transformer block",
 * Code: post-attention RMSNorm, the MLP, then the residual add; the MLP of
 * every block after the first is the MoE, "Kimi K2 · Architecture", Fact
 * sheet: 384 routed + 1 shared experts, 8 chosen per token).
 * Same kernels as the four calls above, with the routing weights applied in
 * the down-projection epilogue; bitwise equal to the unfused chain. */
moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                       const void* w_router, const float* bias, const void* packed_w,
                       void* out, void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a static device array of 48 MiB
 * in the library, one copy per GPU, allocated with the code object and held
 * until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress) on the first call there.  A batch whose
 * moe_workspace_bytes(MOE_WS_FORWARD) exceeds 48 MiB is rejected with
 * MOE_ERR_WORKSPACE (Kimi K2 shape: up to 130 tokens).  No part of the array
 * needs to start zeroed (every workspace word is written before it is read).
 * All calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Results are bitwise those of moe_forward. */
moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x,
                               const void* norm_w, const void* w_router, const float* bias,
                               const void* packed_w, void* out, void* stream);

/* ---- Routing bias update (training): aux-loss-free load balancing.
 *
 * The router adds e_score_correction_bias to the sigmoid scores for the top-k
 * choice only ("Kimi-K2-Base", Mixture of experts, Load balancing; "Kimi K2 ·
 * Architecture", config.json topk_method noaux_tc); the pages state that the
 * rule adjusting that bias is not described.  The rule implemented is the
 * published aux-loss-free balancing rule (Wang et al. 2024): with c_e the
 * number of top-k choices of routed expert e over a training step and cbar
 * = sum_e c_e / E their mean, after the step
 *     bias[e] <- bias[e] + speed * sign(cbar - c_e)      (sign 0 at the mean)
 * with the sign decided exactly on integers and one fp32 addition per expert.
 * A step over several micro-batches accumulates their loads with
 * moe_expert_load into one counts array, then calls moe_bias_update once
 * (with data parallelism the counts are summed over the ranks in between). */

/* counts[e] += number of entries of topk_ids [T, top_k] (int32, from
 * moe_router) equal to e, for 0 <= e < n_experts; other values are not routed
 * experts of this layer and are not counted.  counts: int32 [n_experts],
 * caller-owned device memory, 4-byte aligned, zeroed by the caller at the
 * start of a step; the total over a step must stay below 2^31.  The counts
 * are exact integers, the same whatever order the workgroups add in.  T = 0
 * enqueues nothing; a dense config has no routed experts
 * (MOE_ERR_INVALID_ARG). */
moe_status moe_expert_load(const moe_config* cfg, int64_t T, const int32_t* topk_ids,
                           int32_t* counts, void* stream);

/* bias [n_experts] fp32 (device, in place) <- bias + speed * sign(cbar - c_e)
 * from the step's counts [n_experts] int32 (device); speed must be finite and
 * >= 0 (MOE_ERR_INVALID_ARG otherwise).  Reads counts, writes bias: the
 * counts may be zeroed for the next step once this call has run. */
moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float speed,
                           float* bias, void* stream);

/* ---- diagnostics: per-stage timing with HIP events ---------------------
 * While profiling is on, every entry point records a HIP event before and
 * after each of its kernel stages, on the caller's stream.  This is the only
 * state the library keeps between calls; it is process-wide and guarded by a
 * lock.  moe_profile_read() waits for the recorded events and returns, per
 * stage, the summed elapsed milliseconds and the number of launches since the
 * last reset (arrays of MOE_STAGE_COUNT entries, either may be NULL). */
typedef enum {
  MOE_STAGE_NORM_QUANT = 0,  /* RMSNorm + 1x128 activation quantisation */
  MOE_STAGE_ROUTER_GEMM = 1, /* router logits */
  MOE_STAGE_TOPK = 2,        /* sigmoid, bias, top-k, weights */
  MOE_STAGE_PERMUTE = 3,     /* counts, scans and the stable scatter */
  MOE_STAGE_TILES = 4,       /* m-tile prefix of the grouped GEMMs */
  MOE_STAGE_GATEUP = 5,      /* grouped gate/up GEMM + SwiGLU + requantisation */
  MOE_STAGE_DOWN = 6,        /* grouped down GEMM */
  MOE_STAGE_COMBINE = 7,     /* weighted combine + residual */
  /* the MLA attention entry points of k2mla.h */
  MOE_STAGE_MLA_PROJ = 8,    /* input RMSNorm and quantisation, the four FP8 projections */
  MOE_STAGE_MLA_LATENT = 9,  /* latent norms, cache entries, query absorption */
  MOE_STAGE_MLA_ATTN = 10,   /* attention over the latent cache */
  MOE_STAGE_MLA_VUP = 11,    /* split merge, value up-projection, 1x128 quantisation */
  MOE_STAGE_BALANCE = 12,    /* expert loads and the routing bias update */
  /* the training step of k2train.h */
  MOE_STAGE_TRAIN_FWD = 13,   /* bf16 gate/up (+ FP8 copies) and down GEMMs */
  MOE_STAGE_TRAIN_DGRAD = 14, /* dgrad GEMMs of down and gate/up */
  MOE_STAGE_TRAIN_WGRAD = 15, /* operand transposes and the weight-gradient GEMMs */
  MOE_STAGE_TRAIN_OTHER = 16, /* sums per token, router and RMSNorm backward */
  MOE_STAGE_COUNT = 17
} moe_stage;

moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_read(double* ms, int64_t* launches, int32_t reset);

#ifdef __cplusplus
}
#endif
#endif /* K2MOE_H */
