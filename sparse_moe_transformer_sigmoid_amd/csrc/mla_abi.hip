// C ABI of the MLA attention sub-layer: argument checks, the packed-weight and
// workspace layouts and the launch sequence.  Contract: include/k2mla.h.
#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "k2mla.h"
#include "mla_launch.h"

namespace {

// the error text is the one moe_last_error() returns
std::string& err_text() { return k2::error_text(); }

moe_status fail(moe_status s, const std::string& msg) {
  err_text() = msg;
  return s;
}

#define M_REQUIRE(cond, st, msg) \
  do {                           \
    if (!(cond)) return fail(st, msg); \
  } while (0)

#define M_HIP(expr)                                                            \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return fail(MOE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define M_PTR(p, name)                                                                   \
  do {                                                                                   \
    M_REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");      \
    M_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15u) == 0, MOE_ERR_INVALID_ARG,          \
              std::string(name) + " is not 16-byte aligned");                            \
  } while (0)
#define M_PTR4(p, name)                                                                  \
  do {                                                                                   \
    M_REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");      \
    M_REQUIRE((reinterpret_cast<uintptr_t>(p) & 3u) == 0, MOE_ERR_INVALID_ARG,           \
              std::string(name) + " is not 4-byte aligned");                             \
  } while (0)

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }
int pad256(int n) { return (n + 255) / 256 * 256; }

struct MDims {
  int d, H, ql, kv, nope, rope, v;
  int n_qkv, n_qkv_pad, n_qb, n_o;   // GEMM output widths (qkv padded to 256)
  float eps, smscale;
};

moe_status check_cfg(const mla_config* c, MDims* o) {
  M_REQUIRE(c != nullptr, MOE_ERR_INVALID_ARG, "config is NULL");
  M_REQUIRE(c->d_model > 0 && c->n_heads > 0 && c->q_lora > 0, MOE_ERR_INVALID_ARG,
            "dimensions must be positive");
  M_REQUIRE(c->kv_lora == 512 && c->qk_nope == 128 && c->qk_rope == 64 && c->v_head == 128,
            MOE_ERR_UNSUPPORTED,
            "the kernels implement kv_lora 512, qk_nope 128, qk_rope 64, v_head 128");
  M_REQUIRE(c->n_heads % 16 == 0 && c->n_heads <= 256, MOE_ERR_UNSUPPORTED,
            "n_heads must be a multiple of 16, at most 256");
  M_REQUIRE(c->d_model % 256 == 0 && c->d_model <= 16384, MOE_ERR_UNSUPPORTED,
            "d_model must be a multiple of 256, at most 16384");
  M_REQUIRE(c->q_lora % 256 == 0 && c->q_lora <= 8192, MOE_ERR_UNSUPPORTED,
            "q_lora must be a multiple of 256, at most 8192");
  M_REQUIRE(c->rope_theta > 0.f && c->rope_factor >= 1.f && c->rope_orig_len > 0 &&
                c->beta_fast >= c->beta_slow && c->beta_slow > 0.f,
            MOE_ERR_INVALID_ARG, "invalid rotary parameters");
  M_REQUIRE(c->rms_eps >= 0.f, MOE_ERR_INVALID_ARG, "rms_eps < 0");
  o->d = c->d_model;
  o->H = c->n_heads;
  o->ql = c->q_lora;
  o->kv = c->kv_lora;
  o->nope = c->qk_nope;
  o->rope = c->qk_rope;
  o->v = c->v_head;
  o->n_qkv = o->ql + o->kv + o->rope;
  o->n_qkv_pad = pad256(o->n_qkv);
  o->n_qb = o->H * (o->nope + o->rope);
  o->n_o = o->d;
  o->eps = c->rms_eps;
  const double corr = 0.1 * c->mscale_all_dim * std::log((double)c->rope_factor) + 1.0;
  o->smscale = (float)(corr * corr / std::sqrt((double)(o->nope + o->rope)));
  return MOE_OK;
}

// YaRN frequencies of the rotary pairs: base^(-2i/dim), kept where the original
// context spans more than beta_fast turns, divided by the factor where it spans
// fewer than beta_slow, linear in the number of turns in between
std::vector<double> yarn_inv_freq(const mla_config* c) {
  const int half = c->qk_rope / 2;
  std::vector<double> f(half);
  for (int i = 0; i < half; ++i) {
    const double base = std::pow((double)c->rope_theta, -2.0 * i / c->qk_rope);
    const double turns = c->rope_orig_len * base / (2.0 * M_PI);
    double keep;
    if (c->beta_fast == c->beta_slow)
      keep = turns > c->beta_fast ? 1.0 : 0.0;
    else
      keep = std::min(1.0, std::max(0.0, (turns - c->beta_slow) / (c->beta_fast - c->beta_slow)));
    f[i] = keep * base + (1.0 - keep) * base / c->rope_factor;
  }
  return f;
}

// ---- packed weights: three GEMM matrices in the grouped GEMM's down form,
// the key-value up-projection as bf16 copies of its key rows (transposed, and
// as they are) and value rows with its block scales, the norm weights, the
// frequencies
struct MPacked {
  size_t qkv_codes, qkv_scales, qb_codes, qb_scales, o_codes, o_scales, kvb_scales, ukt, uv, uk,
      g_qa, g_kva, freq, total;
};

MPacked packed_layout(const MDims& D) {
  MPacked p{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += align_up(b);
    return o;
  };
  p.qkv_codes = take((size_t)D.n_qkv_pad * D.d);
  p.qkv_scales = take((size_t)(D.n_qkv_pad / 128) * (D.d / 128) * 4);
  p.qb_codes = take((size_t)D.n_qb * D.ql);
  p.qb_scales = take((size_t)(D.n_qb / 128) * (D.ql / 128) * 4);
  p.o_codes = take((size_t)D.n_o * D.H * D.v);
  p.o_scales = take((size_t)(D.n_o / 128) * D.H * 4);
  p.kvb_scales = take((size_t)D.H * 2 * (D.kv / 128) * 4);
  p.ukt = take((size_t)D.H * D.kv * D.nope * 2);
  p.uv = take((size_t)D.H * D.v * D.kv * 2);
  p.uk = take((size_t)D.H * D.nope * D.kv * 2);
  p.g_qa = take((size_t)D.ql * 2);
  p.g_kva = take((size_t)D.kv * 2);
  p.freq = take((size_t)(D.rope / 2) * 8);
  p.total = off;
  return p;
}

// ---- GEMM launch shape: m-tile width from the batch (at most 64 rows: the
// instances that sum each block product exactly, so the requantised inputs of
// the next projection match an exact evaluation), K slices to fill the chip
int gemm_tt(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }

constexpr int QKV_FUSE_MAX = 2;   // most [q_a; kv_a] K slices the latent kernel adds itself

int gemm_split(int T, int N, int K) {
  const int bm = 16 * gemm_tt(T);
  const int items = ((T + bm - 1) / bm) * (N / 256);
  const int nkb = K / 128;
  int best = 1;
  for (int s = 2; s <= nkb; ++s) {
    if (nkb % s) continue;
    if (nkb / s < 4) break;         // at least 4 K blocks per slice
    if (items * best >= 512) break;
    best = s;
  }
  return best;
}

// attention position splits: a work item per CU (one workgroup fills a CU's LDS), >= 256
// positions each
void attn_split(int T, int H, int n_seq, int n_new, int max_len, int* nsplit, int* chunk) {
  int mode, hw;
  const int items = std::max(1, k2::mla_attn_items(T, H, n_seq, n_new, &mode, &hw));
  int ns = std::max(1, (256 + items - 1) / items);
  ns = std::min(ns, std::max(1, max_len / 256));
  int ch = (max_len + ns - 1) / ns;
  ch = (ch + 31) / 32 * 32;
  *nsplit = (max_len + ch - 1) / ch;
  *chunk = ch;
}

// Prompt-sized batches (at least MHA_MIN_NEW new tokens per sequence) attend
// in the per-head form: forming a position's keys and values costs about as
// much as 150 queries attending to it in the absorbed form, and each query
// then needs 2.4x fewer MFMA products.  Its key-value buffer is bounded.
constexpr int MHA_MIN_NEW = 128;
constexpr size_t MHA_MAX_KV_BYTES = (size_t)1 << 34;

bool use_mha(const MDims& D, int S, int n, int L) {
  return n >= MHA_MIN_NEW && k2::mla_mha_kv_bytes(S, D.H, L) <= MHA_MAX_KV_BYTES;
}

// The output projection of batches of at least O_WIDE_MIN tokens runs in
// 128-row m-tiles with the FP8 MFMA's own block sums: its result goes
// straight to the residual add (no requantisation decides on it), so exact
// block sums buy nothing there.  The same holds for the query up-projection
// when the per-head form consumes its fp32 output directly; the
// [q_a; kv_a] projection keeps exact sums (its latents are normalised and
// requantised, and the absorbed form's queries go through W_uk first).
constexpr int O_WIDE_MIN = 2048;

struct MLayout {
  size_t hbuf, xq, xs, offsets, mt_start, tile_group, mt_start8, tile_group8, part, qkv, qa_q,
      qa_s, qcat, part_o, part_ml, kv, rot, o_q, o_s, total;
  int ns_qkv, ns_qb, ns_o, ns_attn, chunk;
  bool mha, o_wide;
};

MLayout ws_layout(const MDims& D, int S, int n, int L) {
  MLayout w{};
  const size_t T = (size_t)S * n;
  if (T == 0) return w;   // no tokens: nothing enqueued, no workspace
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += align_up(b);
    return o;
  };
  w.ns_qkv = gemm_split((int)T, D.n_qkv_pad, D.d);
  w.ns_qb = gemm_split((int)T, D.n_qb, D.ql);
  w.o_wide = T >= (size_t)O_WIDE_MIN;
  w.ns_o = w.o_wide ? 1 : gemm_split((int)T, D.n_o, D.H * D.v);
  attn_split((int)T, D.H, S, n, L, &w.ns_attn, &w.chunk);
  w.hbuf = take(T * D.d * 2);
  w.xq = take(T * D.d);
  w.xs = take(T * (D.d / 128) * 4);
  w.offsets = take(2 * 4);
  w.mt_start = take(2 * 4);
  w.tile_group = take(((T + 15) / 16 + 1) * 4);
  if (w.o_wide) {
    w.mt_start8 = take(2 * 4);
    w.tile_group8 = take(((T + 127) / 128 + 1) * 4);
  }
  const size_t part_elems = std::max({(size_t)w.ns_qkv * T * D.n_qkv_pad,
                                      (size_t)w.ns_qb * T * D.n_qb, (size_t)w.ns_o * T * D.n_o});
  w.part = take(part_elems * 4);
  // the [q_a; kv_a] K slices are summed by a separate launch when there are
  // many of them (small batches: the latent kernel has one workgroup per
  // token, too few to wait on many slices); otherwise in the latent kernel
  w.qkv = w.ns_qkv > QKV_FUSE_MAX ? take(T * D.n_qkv_pad * 4) : 0;
  w.qa_q = take(T * D.ql);
  w.qa_s = take(T * (D.ql / 128) * 4);
  w.mha = use_mha(D, S, n, L);
  if (w.mha) {
    w.kv = take(k2::mla_mha_kv_bytes(S, D.H, L));
    w.rot = take(T * (D.rope / 2) * 2 * 8);
  } else {
    w.qcat = take(T * D.H * (D.kv + D.rope) * 4);
    w.part_o = take((size_t)w.ns_attn * T * D.H * D.kv * 4);
    w.part_ml = take((size_t)w.ns_attn * T * D.H * 2 * 4);
  }
  w.o_q = take(T * D.H * D.v);
  w.o_s = take(T * D.H * 4);
  w.total = T == 0 ? 0 : off;
  return w;
}

template <class Tp>
Tp* at(void* base, size_t off) {
  return reinterpret_cast<Tp*>(static_cast<uint8_t*>(base) + off);
}

// one dense FP8 projection: out [nsplit, T, N] partial sums of act [T, K] codes
moe_status run_gemm(const MDims& D, int T, int N, int K, int nsplit, const uint8_t* act,
                    const float* act_s, const uint8_t* wcodes, const float* wscales,
                    const int32_t* offsets, const int32_t* mt_start, const int32_t* tile_group,
                    float* out, hipStream_t s, bool wide = false,
                    const uint16_t* res = nullptr, uint16_t* out_bf16 = nullptr) {
  const int tt = wide ? 8 : gemm_tt(T);
  const int bm = 16 * tt;
  k2::GemmArgs a{};
  a.wpk = wcodes;
  a.expert_stride = 0;
  a.wscale = wscales;
  a.wscale_stride = 0;
  a.act = act;
  a.act_s = act_s;
  a.act_ld = K;
  a.nkb = K / 128;
  a.offsets = offsets;
  a.row_pair = offsets;   // read only by the gate/up form and weighted epilogues
  a.mt_start = mt_start;
  a.tile_group = tile_group;
  a.E = 1;
  a.G = 1;
  a.T = T;
  a.k = 1;
  a.P = T;
  a.NC = N / 256;
  a.rows = out;
  a.weighted = 0;
  a.d = N;
  a.res = res;
  a.out_bf16 = out_bf16;
  const int mtiles = (T + bm - 1) / bm;
  const int grid = (mtiles * a.NC + 7) / 8 * 8;
  if (wide)
    M_HIP(k2::launch_gemm_fp8(false, 8, a, grid, s));   // one K slice, FP8 MFMA block sums
  else
    M_HIP(k2::launch_gemm_dense(tt, nsplit, a, grid, s));
  return MOE_OK;
}

moe_status check_call(const mla_config* cfg, int32_t S, int32_t n, int32_t L, MDims* D) {
  moe_status st = check_cfg(cfg, D);
  if (st != MOE_OK) return st;
  M_REQUIRE(S >= 0 && n >= 0 && L > 0, MOE_ERR_INVALID_ARG, "n_seq, n_new >= 0, max_len > 0");
  M_REQUIRE(n <= L, MOE_ERR_INVALID_ARG, "n_new > max_len");
  const int64_t T = (int64_t)S * n;
  M_REQUIRE(T <= (1 << 20) && T * std::max(D->n_qb, D->H * D->kv) * 4 < ((int64_t)1 << 38) &&
                (int64_t)S * L * D->kv < ((int64_t)1 << 40),
            MOE_ERR_UNSUPPORTED, "batch too large");
  M_REQUIRE(T * std::max({D->d, D->ql, D->H * D->v, D->n_qkv_pad, D->n_qb}) < ((int64_t)1 << 31),
            MOE_ERR_UNSUPPORTED, "too many tokens for 32-bit row offsets");
  return MOE_OK;
}

moe_status run_mla(const mla_config* cfg, int32_t S, int32_t n, int32_t L, const void* x,
                   const void* norm_w, const void* packed, const int32_t* cached_len,
                   void* cache_codes, float* cache_scales, void* cache_rope, void* out,
                   bool out_f32, float* attn, void* ws, size_t ws_bytes, hipStream_t s) {
  MDims D;
  moe_status st = check_call(cfg, S, n, L, &D);
  if (st != MOE_OK) return st;
  const int T = S * n;
  if (T == 0) return MOE_OK;
  M_PTR(x, "x");
  M_PTR(norm_w, "norm_w");
  M_PTR(packed, "packed");
  M_PTR4(cached_len, "cached_len");
  M_PTR(cache_codes, "cache_codes");
  M_PTR(cache_scales, "cache_scales");
  M_PTR(cache_rope, "cache_rope");
  if (out) M_PTR(out, "out");
  if (attn) M_PTR(attn, "attn");
  const MLayout W = ws_layout(D, S, n, L);
  M_REQUIRE(ws_bytes >= W.total, MOE_ERR_WORKSPACE, "workspace too small");
  M_PTR(ws, "ws");
  const MPacked P = packed_layout(D);
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  uint8_t* xq = at<uint8_t>(ws, W.xq);
  float* xs = at<float>(ws, W.xs);
  int32_t* offsets = at<int32_t>(ws, W.offsets);
  int32_t* mt_start = at<int32_t>(ws, W.mt_start);
  int32_t* tile_group = at<int32_t>(ws, W.tile_group);
  float* part = at<float>(ws, W.part);
  uint8_t* qa_q = at<uint8_t>(ws, W.qa_q);
  float* qa_s = at<float>(ws, W.qa_s);
  uint16_t* qcat = at<uint16_t>(ws, W.qcat);
  float* part_o = at<float>(ws, W.part_o);
  float* part_ml = at<float>(ws, W.part_ml);
  uint8_t* o_q = at<uint8_t>(ws, W.o_q);
  float* o_s = at<float>(ws, W.o_s);
  const double* freq = reinterpret_cast<const double*>(pk + P.freq);
  const uint16_t* ukt = reinterpret_cast<const uint16_t*>(pk + P.ukt);
  const uint16_t* uv = reinterpret_cast<const uint16_t*>(pk + P.uv);
  const uint16_t* uk = reinterpret_cast<const uint16_t*>(pk + P.uk);
  const float* kvbs = reinterpret_cast<const float*>(pk + P.kvb_scales);

  {
    k2::ProfileScope ps(MOE_STAGE_MLA_PROJ, s);
    // input RMSNorm + 1x128 quantisation
    M_HIP(k2::launch_norm_quant(true, T, D.d, D.eps, x, norm_w, at<void>(ws, W.hbuf), xq, xs,
                                s));
    // the projections' work tables: one group of T rows in m-tiles of
    // 16 gemm_tt(T) rows (the same for all three projections)
    M_HIP(k2::launch_dense_tiles((int)T, 16 * gemm_tt((int)T), offsets, mt_start, tile_group,
                                 s));
    if (W.o_wide)
      M_HIP(k2::launch_dense_tiles((int)T, 128, offsets, at<int32_t>(ws, W.mt_start8),
                                   at<int32_t>(ws, W.tile_group8), s));
    // [q_a; kv_a] = h [W_qa; W_kva]^T
    if ((st = run_gemm(D, T, D.n_qkv_pad, D.d, W.ns_qkv, xq, xs, pk + P.qkv_codes,
                       reinterpret_cast<const float*>(pk + P.qkv_scales), offsets, mt_start,
                       tile_group, part, s)) != MOE_OK)
      return st;
    if (W.ns_qkv > QKV_FUSE_MAX)
      M_HIP(k2::launch_slice_sum(T, D.n_qkv_pad, D.n_qkv_pad, W.ns_qkv, part, nullptr,
                                 at<float>(ws, W.qkv), D.n_qkv_pad, s));
  }
  {
    k2::ProfileScope ps(MOE_STAGE_MLA_LATENT, s);
    // latent norms, query-latent codes, cache entries (few K slices of the
    // projection are added in the kernel)
    const bool fused = W.ns_qkv <= QKV_FUSE_MAX;
    M_HIP(k2::launch_mla_latent(T, fused ? W.ns_qkv : 1, D.ql, D.n_qkv_pad, D.eps,
                                fused ? part : at<float>(ws, W.qkv),
                                reinterpret_cast<const uint16_t*>(pk + P.g_qa),
                                reinterpret_cast<const uint16_t*>(pk + P.g_kva), freq,
                                cached_len, n, L, qa_q, qa_s, static_cast<uint8_t*>(cache_codes),
                                cache_scales, static_cast<uint16_t*>(cache_rope),
                                W.mha ? at<double>(ws, W.rot) : nullptr, s));
  }
  {
    k2::ProfileScope ps(MOE_STAGE_MLA_PROJ, s);
    // q = qa W_qb^T
    const bool qb_wide = W.o_wide && W.mha;
    if ((st = run_gemm(D, T, D.n_qb, D.ql, qb_wide ? 1 : W.ns_qb, qa_q, qa_s, pk + P.qb_codes,
                       reinterpret_cast<const float*>(pk + P.qb_scales), offsets,
                       qb_wide ? at<int32_t>(ws, W.mt_start8) : mt_start,
                       qb_wide ? at<int32_t>(ws, W.tile_group8) : tile_group, part, s,
                       qb_wide)) != MOE_OK)
      return st;
  }
  if (W.mha) {
    // per-head keys and values of every visible position, then attention
    // (the q_b projection's K-slice partial sums are added in the kernel)
    k2::ProfileScope ps(MOE_STAGE_MLA_ATTN, s);
    M_HIP(k2::launch_mla_mha(T, D.H, S, n, L, W.o_wide ? 1 : W.ns_qb, D.smscale, part,
                             at<double>(ws, W.rot), cached_len,
                             static_cast<const uint8_t*>(cache_codes), cache_scales,
                             static_cast<const uint16_t*>(cache_rope), uk, uv, kvbs,
                             at<uint16_t>(ws, W.kv), o_q, o_s, attn, s));
  } else {
    {
      k2::ProfileScope ps(MOE_STAGE_MLA_LATENT, s);
      // absorbed queries
      // (the q_b projection's K-slice partial sums are added in the kernel)
      M_HIP(k2::launch_mla_qabsorb(T, D.H, W.ns_qb, D.smscale, part, ukt, kvbs, freq,
                                   cached_len, n, L, qcat, s));
    }
    {
      k2::ProfileScope ps(MOE_STAGE_MLA_ATTN, s);
      M_HIP(k2::launch_mla_attn(T, D.H, S, n, L, W.ns_attn, W.chunk,
                                static_cast<const uint8_t*>(cache_codes), cache_scales,
                                static_cast<const uint16_t*>(cache_rope), qcat, cached_len,
                                part_o, part_ml, s));
    }
    {
      k2::ProfileScope ps(MOE_STAGE_MLA_VUP, s);
      M_HIP(k2::launch_mla_vup(T, D.H, W.ns_attn, part_o, part_ml, uv, kvbs, o_q, o_s, attn, s));
    }
  }
  if (!out) return MOE_OK;
  k2::ProfileScope ps(MOE_STAGE_MLA_PROJ, s);
  // out = x + o W_o^T; one K slice with a bf16 output: the residual add in
  // the GEMM's epilogue (the same rounding as the slice sum's)
  const bool fused = W.ns_o == 1 && !out_f32;
  if ((st = run_gemm(D, T, D.n_o, D.H * D.v, W.ns_o, o_q, o_s, pk + P.o_codes,
                     reinterpret_cast<const float*>(pk + P.o_scales), offsets,
                     W.o_wide ? at<int32_t>(ws, W.mt_start8) : mt_start,
                     W.o_wide ? at<int32_t>(ws, W.tile_group8) : tile_group, part, s,
                     W.o_wide, fused ? static_cast<const uint16_t*>(x) : nullptr,
                     fused ? static_cast<uint16_t*>(out) : nullptr)) != MOE_OK)
    return st;
  if (!fused)
    M_HIP(k2::launch_slice_sum(T, D.n_o, D.n_o, W.ns_o, part,
                               out_f32 ? nullptr : static_cast<const uint16_t*>(x), out, D.n_o,
                               s));
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t mla_packed_weights_bytes(const mla_config* cfg) {
  MDims D;
  if (check_cfg(cfg, &D) != MOE_OK) return 0;
  return packed_layout(D).total;
}

moe_status mla_pack_weights(const mla_config* cfg, const mla_weights* w, void* packed,
                            void* stream) {
  MDims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  M_REQUIRE(w != nullptr, MOE_ERR_INVALID_ARG, "weights is NULL");
  M_PTR(w->w_qa, "w_qa");
  M_PTR(w->w_qb, "w_qb");
  M_PTR(w->w_kva, "w_kva");
  M_PTR(w->w_kvb, "w_kvb");
  M_PTR(w->w_o, "w_o");
  M_PTR4(w->s_qa, "s_qa");
  M_PTR4(w->s_qb, "s_qb");
  M_PTR4(w->s_kva, "s_kva");
  M_PTR4(w->s_kvb, "s_kvb");
  M_PTR4(w->s_o, "s_o");
  M_PTR4(w->g_qa, "g_qa");
  M_PTR4(w->g_kva, "g_kva");
  M_PTR(packed, "packed");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const MPacked P = packed_layout(D);
  uint8_t* base = static_cast<uint8_t*>(packed);
  auto u8 = [](const void* p) { return static_cast<const uint8_t*>(p); };
  M_HIP(k2::launch_pack_rows(D.n_qkv_pad, D.d, u8(w->w_qa), D.ql, u8(w->w_kva), D.kv + D.rope,
                             w->s_qa, w->s_kva, base + P.qkv_codes,
                             reinterpret_cast<float*>(base + P.qkv_scales), s));
  M_HIP(k2::launch_pack_rows(D.n_qb, D.ql, u8(w->w_qb), D.n_qb, nullptr, 0, w->s_qb, nullptr,
                             base + P.qb_codes, reinterpret_cast<float*>(base + P.qb_scales), s));
  M_HIP(k2::launch_pack_rows(D.n_o, D.H * D.v, u8(w->w_o), D.n_o, nullptr, 0, w->s_o, nullptr,
                             base + P.o_codes, reinterpret_cast<float*>(base + P.o_scales), s));
  M_HIP(k2::launch_mla_pack_ukv(D.H, u8(w->w_kvb), reinterpret_cast<uint16_t*>(base + P.ukt),
                                reinterpret_cast<uint16_t*>(base + P.uv),
                                reinterpret_cast<uint16_t*>(base + P.uk), s));
  M_HIP(hipMemcpyAsync(base + P.kvb_scales, w->s_kvb, (size_t)D.H * 2 * (D.kv / 128) * 4,
                       hipMemcpyDeviceToDevice, s));
  M_HIP(hipMemcpyAsync(base + P.g_qa, w->g_qa, (size_t)D.ql * 2, hipMemcpyDeviceToDevice, s));
  M_HIP(hipMemcpyAsync(base + P.g_kva, w->g_kva, (size_t)D.kv * 2, hipMemcpyDeviceToDevice, s));
  const std::vector<double> f = yarn_inv_freq(cfg);
  M_HIP(hipMemcpyAsync(base + P.freq, f.data(), f.size() * 8, hipMemcpyHostToDevice, s));
  M_HIP(hipStreamSynchronize(s));   // the host frequency table must outlive the copy
  return MOE_OK;
}

moe_status mla_workspace_bytes(const mla_config* cfg, int32_t n_seq, int32_t n_new,
                               int32_t max_len, size_t* bytes) {
  MDims D;
  moe_status st = check_call(cfg, n_seq, n_new, max_len, &D);
  if (st != MOE_OK) return st;
  M_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(D, n_seq, n_new, max_len).total;
  return MOE_OK;
}

moe_status mla_forward(const mla_config* cfg, int32_t n_seq, int32_t n_new, int32_t max_len,
                       const void* x, const void* norm_w, const void* packed,
                       const int32_t* cached_len, void* cache_codes, float* cache_scales,
                       void* cache_rope, void* out, int32_t out_f32, void* ws, size_t ws_bytes,
                       void* stream) {
  M_REQUIRE(out_f32 == 0 || out_f32 == 1, MOE_ERR_INVALID_ARG, "out_f32 must be 0 or 1");
  if ((int64_t)n_seq * n_new > 0)
    M_REQUIRE(out != nullptr, MOE_ERR_INVALID_ARG, "out is NULL");
  return run_mla(cfg, n_seq, n_new, max_len, x, norm_w, packed, cached_len, cache_codes,
                 cache_scales, cache_rope, out, out_f32 != 0, nullptr, ws, ws_bytes,
                 static_cast<hipStream_t>(stream));
}

moe_status mla_attention(const mla_config* cfg, int32_t n_seq, int32_t n_new, int32_t max_len,
                         const void* x, const void* norm_w, const void* packed,
                         const int32_t* cached_len, void* cache_codes, float* cache_scales,
                         void* cache_rope, float* attn, void* ws, size_t ws_bytes,
                         void* stream) {
  if ((int64_t)n_seq * n_new > 0)
    M_REQUIRE(attn != nullptr, MOE_ERR_INVALID_ARG, "attn is NULL");
  return run_mla(cfg, n_seq, n_new, max_len, x, norm_w, packed, cached_len, cache_codes,
                 cache_scales, cache_rope, nullptr, false, attn, ws, ws_bytes,
                 static_cast<hipStream_t>(stream));
}

}  // extern "C"
