/*
 * k2mla.h -- C ABI of Kimi K2's multi-head latent attention (MLA) sub-layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The sub-layer is the attention half of a Kimi K2 decoder block ("Kimi K2 ·
 * Dense transformer block", Code: input RMSNorm, self-attention, residual add):
 *
 *     out = x + W_o MLA(RMSNorm(x))
 *
 * MLA ("Kimi K2 · Architecture", Fact sheet and config.json; "Kimi-K2-Base",
 * Attention): the query comes from a 1,536-wide latent and the keys and values
 * from a 512-wide latent, each RMS-normalised before its up-projection; every
 * head has 128 query/key features without position and 64 rotary ones (one
 * rotary key shared by all heads) and 128 value features; scores are scaled by
 * (0.1 ln 32 + 1)^2 / sqrt(192) (YaRN, factor 32, original context 4096) and
 * causally masked; positions are numbered from the cached length.  All five
 * projection matrices are FP8 e4m3 with 128x128 block scales and dynamically
 * quantised 1x128 activations (config.json quantization_config).
 *
 * Latent cache, one entry per (sequence, position), caller-owned device memory:
 *   codes  [S, max_len, 512] uint8 : e4m3 codes of the normalised latent
 *   scales [S, max_len, 4]   fp32  : their 1x128 scales
 *   rope   [S, max_len, 64]  bf16  : the rotated positional key
 * 656 bytes per position: the latent is cached as the FP8 input of the
 * key-value up-projection (which is what that FP8 linear reads), where a bf16
 * latent takes 1,152 bytes ("Kimi-K2-Base", KV cache: 70,272 B per token over
 * 61 layers).  Two forms of the same attention are used:
 *   - absorbed (decode and small chunks): the query's key part is multiplied
 *     into latent space and the value up-projection is applied after the
 *     weighted sum, so the per-head keys and values are never formed;
 *   - per head (at least 128 new tokens per sequence, key/value buffer at
 *     most 16 GiB): the keys W_uk c and values W_uv c of every visible
 *     position and head are formed in the workspace (1 KiB per position and
 *     head, as bf16 high and low halves) and attended flash-style.
 * mla_workspace_bytes reports the size for the form the call will use.
 *
 * Batch: S sequences, each with the same number n of new tokens (T = S * n;
 * decode: n = 1; prefill: n = prompt length), token t belongs to sequence
 * t / n at position cached_len[t / n] + t % n.  The call writes the new tokens'
 * cache entries and attends over positions 0 .. that position.
 *
 * Conventions as in k2moe.h: device pointers, caller-owned, row-major,
 * 16-byte aligned (scale arrays and cached_len 4-byte); every call enqueues on
 * `stream` and returns without synchronising; arguments are validated on the
 * host before any HIP call; results are deterministic (no floating-point
 * atomics).  T = 0 enqueues nothing.
 */
#ifndef K2MLA_H
#define K2MLA_H

#include <stddef.h>
#include <stdint.h>

#include "k2moe.h"   /* moe_status, moe_last_error, moe_status_str */

#ifdef __cplusplus
extern "C" {
#endif

/* Shape, mirroring config.json (hidden_size, num_attention_heads, q_lora_rank,
 * kv_lora_rank, qk_nope_head_dim, qk_rope_head_dim, v_head_dim, rope_theta,
 * rope_scaling, rms_norm_eps).  The kernels implement kv_lora = 512,
 * qk_nope = 128, qk_rope = 64, v_head = 128, n_heads % 16 == 0,
 * d_model % 256 == 0 and q_lora % 256 == 0 (others: MOE_ERR_UNSUPPORTED). */
typedef struct {
  int32_t d_model;       /* 7168 */
  int32_t n_heads;       /* 64 */
  int32_t q_lora;        /* 1536 */
  int32_t kv_lora;       /* 512 */
  int32_t qk_nope;       /* 128 */
  int32_t qk_rope;       /* 64 */
  int32_t v_head;        /* 128 */
  int32_t rope_orig_len; /* 4096 */
  float rope_theta;      /* 50000 */
  float rope_factor;     /* 32 */
  float beta_fast;       /* 1 */
  float beta_slow;       /* 1 */
  float mscale_all_dim;  /* 1 */
  float rms_eps;         /* 1e-6 */
} mla_config;

/* The weights in canonical layout (device pointers): e4m3 codes in nn.Linear
 * [out, in] layout with fp32 scales [ceil(out/128), in/128], and the two bf16
 * latent-norm weights.
 *   w_qa [q_lora, d_model]            w_qb [heads*(nope+rope), q_lora]
 *   w_kva [kv_lora+rope, d_model]     w_kvb [heads*(nope+v), kv_lora]
 *   w_o [d_model, heads*v]            g_qa [q_lora], g_kva [kv_lora]
 * Head h's query rows are [nope, rope] at h*(nope+rope); its key-value rows
 * are [nope key rows, v value rows] at h*(nope+v). */
typedef struct {
  const void* w_qa;  const float* s_qa;
  const void* w_qb;  const float* s_qb;
  const void* w_kva; const float* s_kva;
  const void* w_kvb; const float* s_kvb;
  const void* w_o;   const float* s_o;
  const void* g_qa;
  const void* g_kva;
} mla_weights;

/* Bytes of the packed weight buffer. */
size_t mla_packed_weights_bytes(const mla_config* cfg);

/* One-time re-layout of the weights into the packed buffer (model-load step):
 * the query and key-value down-projections are stacked and, with the query
 * up-projection and the output projection, cut into the MFMA fragment order
 * of the grouped FP8 GEMM; the key-value up-projection and the norm weights
 * are copied as they are. */
moe_status mla_pack_weights(const mla_config* cfg, const mla_weights* w, void* packed,
                            void* stream);

/* Workspace bytes for a batch of T = n_seq * n_new tokens whose longest
 * attended range is at most max_len positions. */
moe_status mla_workspace_bytes(const mla_config* cfg, int32_t n_seq, int32_t n_new,
                               int32_t max_len, size_t* bytes);

/* The attention sub-layer for T = n_seq * n_new new tokens.
 *  x [T, d_model] bf16; norm_w [d_model] bf16 (input RMSNorm weight);
 *  packed: from mla_pack_weights; cached_len [n_seq] int32 (device): cached
 *  positions of each sequence before this call, with
 *  cached_len + n_new <= max_len (positions past max_len are not checked on
 *  the device: the caller guarantees the bound);
 *  cache_*: the latent cache (layout above), capacity max_len per sequence;
 *  the call writes positions cached_len .. cached_len + n_new - 1;
 *  out [T, d_model]: out_f32 = 0: bf16 x + W_o MLA(RMSNorm(x)) (one rounding);
 *  out_f32 = 1: fp32 W_o MLA(RMSNorm(x)) without the residual. */
moe_status mla_forward(const mla_config* cfg, int32_t n_seq, int32_t n_new, int32_t max_len,
                       const void* x, const void* norm_w, const void* packed,
                       const int32_t* cached_len, void* cache_codes, float* cache_scales,
                       void* cache_rope, void* out, int32_t out_f32, void* ws, size_t ws_bytes,
                       void* stream);

/* The same call, stopping before the output projection: attn [T, heads*v]
 * fp32 is the attention output of every head (the input of W_o). */
moe_status mla_attention(const mla_config* cfg, int32_t n_seq, int32_t n_new, int32_t max_len,
                         const void* x, const void* norm_w, const void* packed,
                         const int32_t* cached_len, void* cache_codes, float* cache_scales,
                         void* cache_rope, float* attn, void* ws, size_t ws_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* K2MLA_H */
