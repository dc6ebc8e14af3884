// C ABI of the K2 MoE layer: argument validation, workspace layout and the
// launch sequence of each entry point.  See include/k2moe.h for the contract.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "k2_launch.h"
#include "k2moe.h"
#include "k2train.h"
#include "train_launch.h"

namespace {

thread_local std::string g_err;

}  // namespace

// detail of the last non-OK status on this host thread, shared by every entry
// point of the library (moe_last_error)
std::string& k2::error_text() { return g_err; }

namespace {

moe_status fail(moe_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define K2_REQUIRE(cond, st, msg) \
  do {                            \
    if (!(cond)) return fail(st, msg); \
  } while (0)

#define K2_HIP(expr)                                                          \
  do {                                                                        \
    hipError_t e_ = (expr);                                                   \
    if (e_ != hipSuccess)                                                     \
      return fail(MOE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// ---- per-stage event profiling (off unless enabled)
struct Profiler {
  std::mutex mu;
  bool on = false;
  struct Rec { int stage; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double ms[MOE_STAGE_COUNT] = {};
  int64_t n[MOE_STAGE_COUNT] = {};

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  // drain recorded pairs into the totals; caller holds mu
  hipError_t drain() {
    hipError_t first = hipSuccess;
    for (const Rec& r : pending) {
      float t = 0.f;
      hipError_t err = hipEventSynchronize(r.b);
      if (err == hipSuccess) err = hipEventElapsedTime(&t, r.a, r.b);
      if (err == hipSuccess) {
        ms[r.stage] += t;
        n[r.stage] += 1;
      } else if (first == hipSuccess) {
        first = err;
      }
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    pending.clear();
    return first;
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// Records an event pair around one stage when profiling is on.
class Stage {
 public:
  Stage(int stage, hipStream_t s) : stage_(stage), s_(s) {
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on) return;
    a_ = p.get();
    b_ = p.get();
    if (a_ && b_ && hipEventRecord(a_, s_) == hipSuccess) active_ = true;
  }
  ~Stage() {
    if (!active_) return;
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (hipEventRecord(b_, s_) == hipSuccess) p.pending.push_back({stage_, a_, b_});
  }

 private:
  int stage_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
};

}  // namespace

// stage timing for the other translation units of the library (the MLA calls)
void* k2::profile_begin(int stage, hipStream_t s) {
  Stage* st = new Stage(stage, s);
  return st;
}
void k2::profile_end(void* handle) { delete static_cast<Stage*>(handle); }

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Dims {
  int d, E, S, k, I, G;
  bool fp8, dense;
  float scaling, eps;
  int renorm;
  int64_t T, P;
};

moe_status check_cfg(const moe_config* c, Dims* o) {
  K2_REQUIRE(c != nullptr, MOE_ERR_INVALID_ARG, "config is NULL");
  K2_REQUIRE(c->fmt == MOE_FMT_F32 || c->fmt == MOE_FMT_BF16_FP8B128, MOE_ERR_UNSUPPORTED,
             "unknown fmt");
  K2_REQUIRE(c->n_group == 1 && c->topk_group == 1, MOE_ERR_UNSUPPORTED,
             "only one expert group (n_group = topk_group = 1) is implemented");
  K2_REQUIRE(c->d_model > 0 && c->d_ff > 0 && c->n_experts > 0 && c->top_k > 0,
             MOE_ERR_INVALID_ARG, "dimensions must be positive");
  K2_REQUIRE(c->top_k <= c->n_experts, MOE_ERR_INVALID_ARG, "top_k > n_experts");
  K2_REQUIRE(c->n_shared == 0 || c->n_shared == 1, MOE_ERR_UNSUPPORTED, "n_shared must be 0 or 1");
  K2_REQUIRE(c->top_k <= 32 && c->n_experts <= 1024, MOE_ERR_UNSUPPORTED,
             "top_k <= 32 and n_experts <= 1024 are supported");
  K2_REQUIRE(c->d_model <= 16384, MOE_ERR_UNSUPPORTED, "d_model <= 16384 is supported");
  K2_REQUIRE(c->d_ff <= 65536, MOE_ERR_UNSUPPORTED, "d_ff <= 65536 is supported");
  K2_REQUIRE(c->dense == 0 || c->dense == 1, MOE_ERR_INVALID_ARG, "dense must be 0 or 1");
  if (c->dense)
    K2_REQUIRE(c->n_experts == 1 && c->top_k == 1 && c->n_shared == 0, MOE_ERR_INVALID_ARG,
               "dense mode needs n_experts = top_k = 1 and n_shared = 0");
  const bool fp8 = c->fmt == MOE_FMT_BF16_FP8B128;
  if (fp8) {
    K2_REQUIRE(c->d_model % 256 == 0 && c->d_ff % 128 == 0, MOE_ERR_UNSUPPORTED,
               "FP8 format needs d_model % 256 == 0 and d_ff % 128 == 0");
    K2_REQUIRE(c->dense || c->n_experts % 16 == 0, MOE_ERR_UNSUPPORTED,
               "FP8 format needs n_experts % 16 == 0");
  } else {
    K2_REQUIRE(c->d_model % 8 == 0, MOE_ERR_UNSUPPORTED, "F32 format needs d_model % 8 == 0");
  }
  K2_REQUIRE(c->rms_eps >= 0.f, MOE_ERR_INVALID_ARG, "rms_eps < 0");
  o->d = c->d_model;
  o->E = c->n_experts;
  o->S = c->n_shared;
  o->k = c->top_k;
  o->I = c->d_ff;
  o->G = o->E + o->S;
  o->fp8 = fp8;
  o->dense = c->dense != 0;
  o->scaling = c->routed_scaling;
  o->eps = c->rms_eps;
  o->renorm = c->norm_topk_prob ? 1 : 0;
  o->T = 0;
  o->P = 0;
  return MOE_OK;
}

moe_status check_tokens(int64_t T, Dims* D) {
  K2_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T < 0");
  const int64_t P = T * D->k;
  const int64_t rows = P + T;
  K2_REQUIRE(T <= (1 << 24) && rows * std::max(D->d, D->I) < (int64_t)1 << 32,
             MOE_ERR_UNSUPPORTED, "too many tokens for 32-bit row offsets");
  D->T = T;
  D->P = P;
  return MOE_OK;
}

#define K2_PTR(p, name)                                                                 \
  do {                                                                                  \
    K2_REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");      \
    K2_REQUIRE(aligned16(p), MOE_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned"); \
  } while (0)
// buffers read or written element by element need only 4-byte alignment
#define K2_PTR4(p, name)                                                                \
  do {                                                                                  \
    K2_REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");      \
    K2_REQUIRE((reinterpret_cast<uintptr_t>(p) & 3u) == 0, MOE_ERR_INVALID_ARG,          \
               std::string(name) + " is not 4-byte aligned");                           \
  } while (0)
#define K2_OPT_PTR4(p, name)                                                            \
  do {                                                                                  \
    K2_REQUIRE((p) == nullptr || (reinterpret_cast<uintptr_t>(p) & 3u) == 0,            \
               MOE_ERR_INVALID_ARG, std::string(name) + " is not 4-byte aligned");      \
  } while (0)
#define K2_OPT_PTR(p, name)                                                             \
  do {                                                                                  \
    K2_REQUIRE((p) == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,                     \
               std::string(name) + " is not 16-byte aligned");                          \
  } while (0)

// router GEMM split over K so small batches still fill the chip
int router_ksplit(const Dims& D) {
  if (!D.fp8 || D.dense) return 1;
  // workgroup tile: 64 tokens x 192 experts; K split in multiples of 128 columns
  const int64_t tiles = ((D.T + 63) / 64) * ((D.E + 191) / 192);
  const int steps = D.d / 128;
  int best = 1;
  for (int ks = 1; ks <= 64; ++ks) {
    if (steps % ks) continue;
    best = ks;
    if (tiles * ks >= 256) break;
  }
  return best;
}

// token tiles (16 rows each) per GEMM m-tile, from the mean rows per group
int gemm_tt(const Dims& D) {
  const double avg = D.dense ? (double)D.T : (double)D.P / D.E;
  if (avg <= 12) return 1;
  if (avg <= 16) return 2;
  if (avg <= 48) return 4;
  return 8;
}

// upper bound of the GEMM m-tiles of a call (the device-side count is exact):
// each non-empty group adds at most bm - 1 padding rows, plus the shared group
int64_t mtile_bound(const Dims& D, int bm) {
  const int64_t nz = std::min<int64_t>(D.E, D.P);
  return (D.P + (int64_t)(bm - 1) * nz) / bm + 1 + (D.S ? ((int64_t)D.T + bm - 1) / bm : 0);
}

struct Layout {
  size_t hbuf = 0, xq = 0, xs = 0, zpart = 0, ids = 0, w = 0, gap = 0, ccount = 0, cbase = 0,
         offsets = 0, row_pair = 0, pair_row = 0, mt_start = 0, tile_group = 0, aq = 0, as = 0,
         rows = 0, shared = 0, total = 0;
  int ksplit = 1, nchunk = 1;
};

// offsets of the workspace sub-buffers each entry point uses
Layout layout(const Dims& D, int entry) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)D.T, P = (size_t)D.P, d = (size_t)D.d, I = (size_t)D.I;
  const size_t E = (size_t)D.E;
  L.ksplit = router_ksplit(D);
  const int chunk = k2::perm_chunk_tokens(D.E);
  L.nchunk = (int)((D.T + chunk - 1) / chunk);
  const bool fwd = entry == MOE_WS_FORWARD;
  if (fwd) {
    L.xq = take(T * d * (D.fp8 ? 1 : 4));
    if (D.fp8) L.xs = take(T * (d / 128) * 4);
    L.ids = take(P * 4);
    L.w = take(P * 4);
    L.gap = take(T * 4);
    L.offsets = take((E + 1) * 4);
    L.row_pair = take(P * 4);
    L.pair_row = take(P * 4);
    L.rows = take(P * d * 4);
    if (D.S) L.shared = take(T * d * 4);
  }
  if (fwd || entry == MOE_WS_ROUTER) {
    if (D.fp8) L.hbuf = take(T * d * 2);
    if (!D.dense) L.zpart = take((size_t)L.ksplit * T * E * 4);
  }
  if (fwd || entry == MOE_WS_PERMUTE) {
    L.ccount = take((size_t)L.nchunk * E * 4);
    L.cbase = take((size_t)L.nchunk * E * 4);
  }
  if (fwd || entry == MOE_WS_SWIGLU) {
    L.mt_start = take(((size_t)D.G + 1) * 4);
    if (D.fp8) L.tile_group = take((size_t)mtile_bound(D, 16 * gemm_tt(D)) * 4);
    const size_t nrows = P + (D.S ? T : 0);
    if (D.fp8) {
      L.aq = take(nrows * I);
      L.as = take(nrows * (I / 128) * 4);
    } else {
      L.aq = take(nrows * I * 4);
    }
  }
  L.total = D.T == 0 ? 0 : off;  // no tokens, nothing enqueued, no workspace
  return L;
}

struct Packed {
  size_t expert_bytes, gu_scale_off, dn_scale_off, gu_scale_floats, dn_scale_floats, total;
};

Packed packed_layout(const Dims& D) {
  Packed p{};
  const size_t NE = (size_t)D.G, d = (size_t)D.d, I = (size_t)D.I;
  if (D.fp8) {
    p.expert_bytes = 3 * I * d;
    p.gu_scale_floats = (I / 128) * (d / 128) * 2;
    p.dn_scale_floats = (d / 128) * (I / 128);
    p.gu_scale_off = align_up(NE * p.expert_bytes);
    p.dn_scale_off = p.gu_scale_off + align_up(NE * p.gu_scale_floats * 4);
    p.total = p.dn_scale_off + align_up(NE * p.dn_scale_floats * 4);
  } else {
    p.expert_bytes = 3 * I * d * 4;
    p.total = NE * p.expert_bytes;
  }
  return p;
}

template <class Tp>
Tp* at(void* base, size_t off) {
  return reinterpret_cast<Tp*>(static_cast<uint8_t*>(base) + off);
}

// ---- launch sequences shared by the unfused entry points and moe_forward

moe_status run_router(const Dims& D, const Layout& L, void* ws, const void* x, const void* norm_w,
                      const void* w_router, const float* bias, int32_t* ids, float* w, float* gap,
                      void* xq, float* xs, hipStream_t s) {
  const int T = (int)D.T;
  void* hbuf = D.fp8 ? at<void>(ws, L.hbuf) : nullptr;
  {
    Stage st(MOE_STAGE_NORM_QUANT, s);
    K2_HIP(k2::launch_norm_quant(D.fp8, T, D.d, D.eps, x, norm_w, hbuf, xq, xs, s));
  }
  if (D.dense) {
    Stage st(MOE_STAGE_TOPK, s);
    K2_HIP(k2::launch_dense_route(T, D.scaling, ids, w, gap, s));
    return MOE_OK;
  }
  float* zpart = at<float>(ws, L.zpart);
  {
  Stage st(MOE_STAGE_ROUTER_GEMM, s);
  if (D.fp8)
    K2_HIP(k2::launch_router_gemm_bf16(T, D.d, D.E, L.ksplit, static_cast<const uint16_t*>(hbuf),
                                       static_cast<const uint16_t*>(w_router), zpart, s));
  else
    K2_HIP(k2::launch_router_gemm_f32(T, D.d, D.E, static_cast<const float*>(xq),
                                      static_cast<const float*>(w_router), zpart, s));
  }
  Stage st(MOE_STAGE_TOPK, s);
  K2_HIP(k2::launch_topk(T, D.E, D.k, D.fp8 ? L.ksplit : 1, zpart, bias, D.scaling, D.renorm,
                         ids, w, gap, s));
  return MOE_OK;
}

moe_status run_permute(const Dims& D, const Layout& L, void* ws, const int32_t* ids,
                       int32_t* offsets, int32_t* row_pair, int32_t* pair_row, hipStream_t s,
                       const k2::TileReq* tiles = nullptr, bool* tiles_built = nullptr) {
  Stage st(MOE_STAGE_PERMUTE, s);
  K2_HIP(k2::launch_permute((int)D.T, D.E, D.k, ids, at<int32_t>(ws, L.ccount),
                            at<int32_t>(ws, L.cbase), offsets, row_pair, pair_row, s, tiles,
                            tiles_built));
  return MOE_OK;
}

moe_status run_experts(const Dims& D, const Layout& L, void* ws, const void* xq, const float* xs,
                       const int32_t* offsets, const int32_t* row_pair, const void* packed_w,
                       float* rows, float* shared_out, const float* topk_w, int weighted,
                       void* act_q, float* act_s, hipStream_t s, bool tiles_ready = false) {
  const int T = (int)D.T, P = (int)D.P;
  const Packed pk = packed_layout(D);
  if (!D.fp8) {
    Stage st(MOE_STAGE_GATEUP, s);
    K2_HIP(k2::launch_experts_f32(T, D.d, D.I, D.E, D.k, D.S, static_cast<const float*>(xq),
                                  offsets, row_pair, static_cast<const float*>(packed_w),
                                  pk.expert_bytes / 4, at<float>(ws, L.aq), rows, shared_out,
                                  topk_w, weighted, s));
    return MOE_OK;
  }
  const int tt = gemm_tt(D);
  const int bm = 16 * tt;
  int32_t* mt_start = at<int32_t>(ws, L.mt_start);
  int32_t* tile_group = at<int32_t>(ws, L.tile_group);
  const int64_t mt_bound = mtile_bound(D, bm);
  if (!tiles_ready) {
    Stage st(MOE_STAGE_TILES, s);
    K2_HIP(k2::launch_build_tiles(D.E, D.S, T, D.k, bm, (int)mt_bound, offsets, mt_start,
                                  tile_group, s));
  }
  auto grid_of = [&](int nc) {
    const int64_t g = (mt_bound * nc + 7) / 8 * 8;
    return (int)std::min<int64_t>(g, (int64_t)1 << 30);
  };
  uint8_t* aq = act_q ? static_cast<uint8_t*>(act_q) : at<uint8_t>(ws, L.aq);
  float* as = act_s ? act_s : at<float>(ws, L.as);
  const uint8_t* pw = static_cast<const uint8_t*>(packed_w);

  k2::GemmArgs a{};
  a.offsets = offsets;
  a.row_pair = row_pair;
  a.mt_start = mt_start;
  a.tile_group = tile_group;
  a.E = D.E;
  a.G = D.G;
  a.T = T;
  a.k = D.k;
  a.P = P;
  a.aq = aq;
  a.as = as;
  a.I = D.I;
  a.rows = rows;
  a.shared_out = shared_out;
  a.topk_w = topk_w;
  a.weighted = weighted;
  a.d = D.d;

  // gate/up + SwiGLU + requantisation: K = d, 128 hidden (256 weight rows) per chunk
  a.wpk = pw;
  a.expert_stride = pk.expert_bytes;
  a.wscale = reinterpret_cast<const float*>(pw + pk.gu_scale_off);
  a.wscale_stride = pk.gu_scale_floats;
  a.act = static_cast<const uint8_t*>(xq);
  a.act_s = xs;
  a.act_ld = D.d;
  a.nkb = D.d / 128;
  a.NC = D.I / 128;
  {
    Stage st(MOE_STAGE_GATEUP, s);
    K2_HIP(k2::launch_gemm_fp8(true, tt, a, grid_of(a.NC), s));
  }

  // down projection: K = I, 256 output rows per chunk
  a.wpk = pw + 2 * (size_t)D.I * D.d;
  a.wscale = reinterpret_cast<const float*>(pw + pk.dn_scale_off);
  a.wscale_stride = pk.dn_scale_floats;
  a.act = aq;
  a.act_s = as;
  a.act_ld = D.I;
  a.nkb = D.I / 128;
  a.NC = D.d / 256;
  {
    Stage st(MOE_STAGE_DOWN, s);
    K2_HIP(k2::launch_gemm_fp8(false, tt, a, grid_of(a.NC), s));
  }
  return MOE_OK;
}

// ---- the training step (k2train.h)

moe_status check_train_cfg(const moe_config* cfg, Dims* D) {
  moe_status st = check_cfg(cfg, D);
  if (st != MOE_OK) return st;
  K2_REQUIRE(D->fp8 && !D->dense, MOE_ERR_UNSUPPORTED,
             "the training step needs fmt = MOE_FMT_BF16_FP8B128 and a routed layer");
  K2_REQUIRE(D->d % 256 == 0 && D->I % 256 == 0, MOE_ERR_UNSUPPORTED,
             "the training step needs d_model % 256 == 0 and d_ff % 256 == 0");
  return MOE_OK;
}

struct TrainSaved {
  size_t hq, hs, ids, w, s, offsets, row_pair, pair_row, guq, gus, total;
};

TrainSaved train_saved(const Dims& D) {
  TrainSaved v{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)D.T, P = (size_t)D.P, d = (size_t)D.d, I = (size_t)D.I;
  const size_t R = P + (D.S ? T : 0);
  v.hq = take(T * d);
  v.hs = take(T * (d / 128) * 4);
  v.ids = take(P * 4);
  v.w = take(P * 4);
  v.s = take(P * 4);
  v.offsets = take(((size_t)D.E + 1) * 4);
  v.row_pair = take(P * 4);
  v.pair_row = take(P * 4);
  v.guq = take(R * 2 * I);
  v.gus = take(R * (2 * I / 128) * 4);
  v.total = D.T == 0 ? 0 : off;
  return v;
}

// Columns of the transposed, group-padded operands of the weight gradients:
// every group pads to a multiple of 32 rows; the grid of the transposes
// covers whole 64-column blocks.
int64_t train_ldt(const Dims& D) {
  const int64_t R = D.P + (D.S ? D.T : 0);
  return (R + 32 * (int64_t)D.G + 63) / 64 * 64;
}

struct TrainLayout {
  Layout fl;   // router / permutation sub-buffers of the forward layout
  size_t gap, mt_start, tile_group, abf, rows, shared, dgu, dwp, dh, dz, dht, colsum, pad_off,
      dywT, aT, dguT, hT, total;
};

TrainLayout train_layout(const Dims& D) {
  TrainLayout L{};
  L.fl = layout(D, MOE_WS_ROUTER);
  const Layout pl = layout(D, MOE_WS_PERMUTE);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  // the router and permutation buffers first, at the offsets those layouts use
  L.fl.ccount = L.fl.total + pl.ccount;
  L.fl.cbase = L.fl.total + pl.cbase;
  off = L.fl.total + pl.total;
  const size_t T = (size_t)D.T, P = (size_t)D.P, d = (size_t)D.d, I = (size_t)D.I;
  const size_t R = P + (D.S ? T : 0);
  const size_t ldt = (size_t)train_ldt(D);
  L.gap = take(T * 4);
  L.mt_start = take(((size_t)D.G + 1) * 4);
  L.tile_group = take((size_t)mtile_bound(D, 128) * 4);
  L.abf = take(R * I * 2);
  L.rows = take(P * d * 4);
  L.shared = take((D.S ? T : 1) * d * 4);
  L.dgu = take(R * 2 * I * 2);
  L.dwp = take(R * (I / 256) * 4);
  L.dh = take(T * d * 4);
  L.dz = take(P * 4);
  L.dht = take(T * d * 4);
  L.colsum = take(k2::col_sum_scratch_bytes((int)D.T, D.d));
  L.pad_off = take(((size_t)D.G + 1) * 4);
  L.dywT = take(d * ldt * 2);
  L.aT = take(I * ldt * 2);
  L.dguT = take(2 * I * ldt * 2);
  L.hT = take(d * ldt * 2);
  L.total = D.T == 0 ? 0 : off;
  return L;
}

int train_grid(const Dims& D, int nc) {
  const int64_t g = (mtile_bound(D, 128) * nc + 7) / 8 * 8;
  return (int)std::min<int64_t>(g, (int64_t)1 << 30);
}

k2::TrainGemmArgs train_rows_args(const Dims& D, const TrainLayout& L, void* ws,
                                  const int32_t* offsets, const int32_t* row_pair) {
  k2::TrainGemmArgs a{};
  a.offsets = offsets;
  a.row_pair = row_pair;
  a.mt_start = at<int32_t>(ws, L.mt_start);
  a.tile_group = at<int32_t>(ws, L.tile_group);
  a.E = D.E;
  a.G = D.G;
  a.T = (int)D.T;
  a.P = (int)D.P;
  a.k = D.k;
  a.I = D.I;
  return a;
}

// ---- the allocation-free forward (moe_forward_noalloc): its workspace is a
// static device array, one copy per GPU, held until the process ends.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)48 << 20;   // K2 shape: up to 130 tokens
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[MAX_DEVICES] = {};

// The device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy; the host-side name is only a handle).
moe_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  K2_HIP(hipGetDevice(&dev));
  K2_REQUIRE(dev >= 0 && dev < MAX_DEVICES, MOE_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    K2_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    K2_REQUIRE(p != nullptr, MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return MOE_OK;
}

// A second stream (default priority) and its events per device, created on
// first use and kept until the process ends: the training backward runs its
// two independent chains on them (fork: the side stream starts; mid: the
// side stream's transposes are done; join: the side chain is done).
struct SideStream {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, mid = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[MAX_DEVICES];

moe_status side_stream_of_current_device(SideStream* out) {
  int dev = -1;
  K2_HIP(hipGetDevice(&dev));
  K2_REQUIRE(dev >= 0 && dev < MAX_DEVICES, MOE_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> g(g_side_mu);
  SideStream& ss = g_side[dev];
  if (ss.s2 == nullptr) {
    SideStream n;
    K2_HIP(hipStreamCreateWithFlags(&n.s2, hipStreamNonBlocking));
    K2_HIP(hipEventCreateWithFlags(&n.fork, hipEventDisableTiming));
    K2_HIP(hipEventCreateWithFlags(&n.mid, hipEventDisableTiming));
    K2_HIP(hipEventCreateWithFlags(&n.join, hipEventDisableTiming));
    ss = n;
  }
  *out = ss;
  return MOE_OK;
}

// The weight gradients of the training backward: the group-padded K-blocked
// transposes of their operands (train_wgrad_transposes), then dW_down and
// dW_gate, dW_up (train_wgrad_gemm), each enqueued on the stream given.
moe_status train_wgrad_transposes(const Dims& D, const TrainLayout& L, int64_t T, void* ws,
                                  void* sv, const TrainSaved& v, const int32_t* offsets,
                                  const int32_t* row_pair, const float* wts, const void* dout,
                                  const uint16_t* abf, const uint16_t* dgu, hipStream_t s) {
  const int64_t ldt = train_ldt(D);
  Stage stg(MOE_STAGE_TRAIN_WGRAD, s);
  int32_t* pad_off = at<int32_t>(ws, L.pad_off);
  K2_HIP(k2::launch_pad_offsets(D.E, D.G, (int)T, (int)D.P, offsets, pad_off, s));
  k2::TransposeArgs ta{};
  ta.offsets = offsets;
  ta.row_pair = row_pair;
  ta.topk_w = wts;
  ta.pad_off = pad_off;
  ta.E = D.E;
  ta.G = D.G;
  ta.T = (int)T;
  ta.P = (int)D.P;
  ta.k = D.k;
  ta.ldt = (int)ldt;
  uint16_t* dywT = at<uint16_t>(ws, L.dywT);
  uint16_t* aT = at<uint16_t>(ws, L.aT);
  uint16_t* dguT = at<uint16_t>(ws, L.dguT);
  uint16_t* hT = at<uint16_t>(ws, L.hT);
  ta.src = static_cast<const uint16_t*>(dout);
  ta.C = D.d;
  ta.dst = dywT;
  K2_HIP(k2::launch_transpose_pad(1, ta, (int)ldt, s));
  ta.src = abf;
  ta.C = D.I;
  ta.dst = aT;
  K2_HIP(k2::launch_transpose_pad(0, ta, (int)ldt, s));
  ta.src = dgu;
  ta.C = 2 * D.I;
  ta.dst = dguT;
  K2_HIP(k2::launch_transpose_pad(0, ta, (int)ldt, s));
  ta.src = nullptr;
  ta.codes = at<const uint8_t>(sv, v.hq);
  ta.scales = at<const float>(sv, v.hs);
  ta.C = D.d;
  ta.dst = hT;
  K2_HIP(k2::launch_transpose_pad(2, ta, (int)ldt, s));
  return MOE_OK;
}

// down: dW_down [d, I] = sum (w dy)^T a~; otherwise dW_gate, dW_up [2I, d] =
// sum [dg; du]^T h~ (after train_wgrad_transposes)
moe_status train_wgrad_gemm(const Dims& D, const TrainLayout& L, void* ws, bool down, float* d_w,
                            hipStream_t s) {
  const size_t d = (size_t)D.d, I = (size_t)D.I;
  Stage stg(MOE_STAGE_TRAIN_WGRAD, s);
  const int32_t* pad_off = at<int32_t>(ws, L.pad_off);
  const uint16_t* dywT = at<uint16_t>(ws, L.dywT);
  const uint16_t* aT = at<uint16_t>(ws, L.aT);
  const uint16_t* dguT = at<uint16_t>(ws, L.dguT);
  const uint16_t* hT = at<uint16_t>(ws, L.hT);
  k2::TrainGemmArgs g{};
  g.E = D.E;
  g.G = D.G;
  g.pad_off = pad_off;
  g.out_stride = 3 * I * d;
  g.A = dywT;   // K-blocked transposed operands: 32 C elements per K block
  g.lda = 32 * D.d;
  g.B = aT;
  g.ldb = 32 * D.I;
  g.MT = D.d / k2::WGRAD_M;
  g.NT = D.I / 128;
  g.out = d_w + 2 * I * d;
  g.ldo = D.I;
  if (down) {
    K2_HIP(k2::launch_train_gemm(k2::TM_WGRAD, g, (D.G * g.MT * g.NT + 7) / 8 * 8, s));
    return MOE_OK;
  }
  g.A = dguT;
  g.lda = 32 * 2 * D.I;
  g.B = hT;
  g.ldb = 32 * D.d;
  g.MT = 2 * D.I / k2::WGRAD_M;
  g.NT = D.d / 128;
  g.out = d_w;
  g.ldo = D.d;
  K2_HIP(k2::launch_train_gemm(k2::TM_WGRAD, g, (D.G * g.MT * g.NT + 7) / 8 * 8, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_profile_enable(int32_t on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return MOE_OK;
}

moe_status moe_profile_read(double* ms, int64_t* launches, int32_t reset) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  const hipError_t err = p.drain();
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) {
    if (ms) ms[i] = p.ms[i];
    if (launches) launches[i] = p.n[i];
  }
  if (reset) {
    for (int i = 0; i < MOE_STAGE_COUNT; ++i) {
      p.ms[i] = 0.0;
      p.n[i] = 0;
    }
  }
  if (err != hipSuccess)
    return fail(MOE_ERR_HIP, std::string("profile events: ") + hipGetErrorString(err));
  return MOE_OK;
}

size_t moe_packed_weights_bytes(const moe_config* cfg) {
  Dims D;
  if (check_cfg(cfg, &D) != MOE_OK) return 0;
  return packed_layout(D).total;
}

moe_status moe_workspace_bytes(const moe_config* cfg, int64_t T, int32_t entry, size_t* bytes) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  K2_REQUIRE(entry >= MOE_WS_ROUTER && entry <= MOE_WS_FORWARD, MOE_ERR_INVALID_ARG,
             "unknown workspace entry");
  K2_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(D, entry).total;
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_config* cfg, const moe_expert_w* experts,
                            int32_t n_experts_total, void* packed, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  K2_REQUIRE(experts != nullptr, MOE_ERR_INVALID_ARG, "experts is NULL");
  K2_REQUIRE(n_experts_total == D.G, MOE_ERR_INVALID_ARG,
             "n_experts_total must be n_experts + n_shared");
  K2_PTR(packed, "packed");
  for (int e = 0; e < D.G; ++e) {
    const moe_expert_w& x = experts[e];
    const std::string nm = "expert " + std::to_string(e) + " ";
    K2_PTR(x.w_gate, nm + "w_gate");
    K2_PTR(x.w_up, nm + "w_up");
    K2_PTR(x.w_down, nm + "w_down");
    if (D.fp8) {
      K2_PTR4(x.s_gate, nm + "s_gate");
      K2_PTR4(x.s_up, nm + "s_up");
      K2_PTR4(x.s_down, nm + "s_down");
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Packed pk = packed_layout(D);
  uint8_t* base = static_cast<uint8_t*>(packed);
  for (int e = 0; e < D.G; ++e) {
    const moe_expert_w& x = experts[e];
    if (D.fp8) {
      K2_HIP(k2::launch_pack_fp8(
          D.d, D.I, static_cast<const uint8_t*>(x.w_gate), static_cast<const uint8_t*>(x.w_up),
          static_cast<const uint8_t*>(x.w_down), x.s_gate, x.s_up, x.s_down,
          base + e * pk.expert_bytes,
          reinterpret_cast<float*>(base + pk.gu_scale_off) + e * pk.gu_scale_floats,
          reinterpret_cast<float*>(base + pk.dn_scale_off) + e * pk.dn_scale_floats, s));
    } else {
      const size_t mat = (size_t)D.I * D.d * 4;
      uint8_t* dst = base + e * pk.expert_bytes;
      K2_HIP(hipMemcpyAsync(dst, x.w_gate, mat, hipMemcpyDeviceToDevice, s));
      K2_HIP(hipMemcpyAsync(dst + mat, x.w_up, mat, hipMemcpyDeviceToDevice, s));
      K2_HIP(hipMemcpyAsync(dst + 2 * mat, x.w_down, mat, hipMemcpyDeviceToDevice, s));
    }
  }
  return MOE_OK;
}

moe_status moe_router(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                      const void* w_router, const float* bias, int32_t* topk_ids, float* topk_w,
                      float* gap, void* xq, float* xs, void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(x, "x");
  K2_PTR(norm_w, "norm_w");
  if (!D.dense) {
    K2_PTR(w_router, "w_router");
    K2_PTR4(bias, "bias");
  }
  K2_PTR4(topk_ids, "topk_ids");
  K2_PTR4(topk_w, "topk_w");
  K2_OPT_PTR4(gap, "gap");
  K2_PTR(xq, "xq");
  if (D.fp8) K2_PTR4(xs, "xs");
  else K2_REQUIRE(xs == nullptr, MOE_ERR_INVALID_ARG, "xs must be NULL in the F32 format");
  const Layout L = layout(D, MOE_WS_ROUTER);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small");
  if (L.total) K2_PTR(ws, "ws");
  if (T == 0) return MOE_OK;
  return run_router(D, L, ws, x, norm_w, w_router, bias, topk_ids, topk_w, gap, xq, xs,
                    static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* row_pair, int32_t* pair_row, void* ws,
                       size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR4(topk_ids, "topk_ids");
  K2_PTR4(expert_offsets, "expert_offsets");
  K2_PTR4(row_pair, "row_pair");
  K2_PTR4(pair_row, "pair_row");
  const Layout L = layout(D, MOE_WS_PERMUTE);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small");
  if (L.total) K2_PTR(ws, "ws");
  if (T == 0) return MOE_OK;
  return run_permute(D, L, ws, topk_ids, expert_offsets, row_pair, pair_row,
                     static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_swiglu(const moe_config* cfg, int64_t T, const void* xq, const float* xs,
                              const int32_t* expert_offsets, const int32_t* row_pair,
                              const void* packed_w, float* rows, float* shared_out, void* act_q,
                              float* act_s, void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(xq, "xq");
  if (D.fp8) K2_PTR4(xs, "xs");
  K2_PTR4(expert_offsets, "expert_offsets");
  K2_PTR4(row_pair, "row_pair");
  K2_PTR(packed_w, "packed_w");
  K2_PTR(rows, "rows");
  if (D.S) K2_PTR(shared_out, "shared_out");
  else K2_REQUIRE(shared_out == nullptr, MOE_ERR_INVALID_ARG,
                  "shared_out must be NULL without a shared expert");
  K2_REQUIRE((act_q == nullptr) == (act_s == nullptr), MOE_ERR_INVALID_ARG,
             "act_q and act_s go together");
  K2_REQUIRE(act_q == nullptr || D.fp8, MOE_ERR_INVALID_ARG,
             "act_q / act_s exist only in the FP8 format");
  K2_OPT_PTR(act_q, "act_q");
  K2_OPT_PTR4(act_s, "act_s");
  const Layout L = layout(D, MOE_WS_SWIGLU);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small");
  if (L.total) K2_PTR(ws, "ws");
  if (T == 0) return MOE_OK;
  return run_experts(D, L, ws, xq, xs, expert_offsets, row_pair, packed_w, rows, shared_out,
                     nullptr, 0, act_q, act_s, static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_config* cfg, int64_t T, const float* rows,
                       const int32_t* pair_row, const float* topk_w, const float* shared_out,
                       const void* residual, void* out, int32_t out_f32, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(rows, "rows");
  K2_PTR4(pair_row, "pair_row");
  K2_PTR4(topk_w, "topk_w");
  if (D.S) K2_PTR(shared_out, "shared_out");
  else K2_REQUIRE(shared_out == nullptr, MOE_ERR_INVALID_ARG,
                  "shared_out must be NULL without a shared expert");
  K2_OPT_PTR(residual, "residual");
  K2_PTR(out, "out");
  K2_REQUIRE(out_f32 == 0 || out_f32 == 1, MOE_ERR_INVALID_ARG, "out_f32 must be 0 or 1");
  if (T == 0) return MOE_OK;
  Stage stg(MOE_STAGE_COMBINE, static_cast<hipStream_t>(stream));
  K2_HIP(k2::launch_combine(D.fp8, !D.fp8 || out_f32, (int)T, D.d, D.k, rows, pair_row, topk_w,
                            1, shared_out, residual, out, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                       const void* w_router, const float* bias, const void* packed_w, void* out,
                       void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(x, "x");
  K2_PTR(norm_w, "norm_w");
  if (!D.dense) {
    K2_PTR(w_router, "w_router");
    K2_PTR4(bias, "bias");
  }
  K2_PTR(packed_w, "packed_w");
  K2_PTR(out, "out");
  const Layout L = layout(D, MOE_WS_FORWARD);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small");
  if (L.total) K2_PTR(ws, "ws");
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* xq = at<void>(ws, L.xq);
  float* xs = D.fp8 ? at<float>(ws, L.xs) : nullptr;
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* w = at<float>(ws, L.w);
  float* gap = at<float>(ws, L.gap);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_pair = at<int32_t>(ws, L.row_pair);
  int32_t* pair_row = at<int32_t>(ws, L.pair_row);
  float* rows = at<float>(ws, L.rows);
  float* shared = D.S ? at<float>(ws, L.shared) : nullptr;
  if ((st = run_router(D, L, ws, x, norm_w, w_router, bias, ids, w, gap, xq, xs, s)) != MOE_OK)
    return st;
  // the FP8 GEMMs' m-tile table, built by the permutation itself when all
  // tokens fit one chunk (decode-sized batches)
  k2::TileReq treq{};
  bool tiles_ready = false;
  if (D.fp8) {
    treq.bm = 16 * gemm_tt(D);
    treq.max_tiles = (int)mtile_bound(D, treq.bm);
    treq.n_shared = D.S;
    treq.mt_start = at<int32_t>(ws, L.mt_start);
    treq.tile_group = at<int32_t>(ws, L.tile_group);
  }
  if ((st = run_permute(D, L, ws, ids, offsets, row_pair, pair_row, s, D.fp8 ? &treq : nullptr,
                        &tiles_ready)) != MOE_OK)
    return st;
  if ((st = run_experts(D, L, ws, xq, xs, offsets, row_pair, packed_w, rows, shared, w, 1,
                        nullptr, nullptr, s, tiles_ready)) !=
      MOE_OK)
    return st;
  Stage stg(MOE_STAGE_COMBINE, s);
  K2_HIP(k2::launch_combine(D.fp8, !D.fp8, (int)T, D.d, D.k, rows, pair_row, w, 0, shared, x, out,
                            s));
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x,
                               const void* norm_w, const void* w_router, const float* bias,
                               const void* packed_w, void* out, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const size_t need = layout(D, MOE_WS_FORWARD).total;
  K2_REQUIRE(need <= NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
             "moe_forward_noalloc: " + std::to_string(T) + " tokens need " +
                 std::to_string(need) + " bytes of workspace; the static scratch array holds " +
                 std::to_string(NOALLOC_SCRATCH_BYTES) + " (Kimi K2 shape: up to 130 tokens)");
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  return moe_forward(cfg, T, x, norm_w, w_router, bias, packed_w, out, ws, need, stream);
}

moe_status moe_expert_load(const moe_config* cfg, int64_t T, const int32_t* topk_ids,
                           int32_t* counts, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  K2_REQUIRE(!D.dense, MOE_ERR_INVALID_ARG, "a dense layer has no routed experts to balance");
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR4(topk_ids, "topk_ids");
  K2_PTR4(counts, "counts");
  Stage stg(MOE_STAGE_BALANCE, static_cast<hipStream_t>(stream));
  K2_HIP(k2::launch_expert_load(D.P, D.E, topk_ids, counts, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float speed,
                           float* bias, void* stream) {
  Dims D;
  moe_status st = check_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  K2_REQUIRE(!D.dense, MOE_ERR_INVALID_ARG, "a dense layer has no routing bias");
  K2_REQUIRE(std::isfinite(speed) && speed >= 0.f, MOE_ERR_INVALID_ARG,
             "speed must be finite and >= 0");
  K2_PTR4(counts, "counts");
  K2_PTR4(bias, "bias");
  Stage stg(MOE_STAGE_BALANCE, static_cast<hipStream_t>(stream));
  K2_HIP(k2::launch_bias_update(D.E, counts, speed, bias, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

size_t moe_train_weights_bytes(const moe_config* cfg) {
  Dims D;
  if (check_train_cfg(cfg, &D) != MOE_OK) return 0;
  return (size_t)D.G * 3 * (size_t)D.I * D.d * 2;
}

size_t moe_train_transposed_bytes(const moe_config* cfg) {
  return moe_train_weights_bytes(cfg);
}

moe_status moe_train_transpose_weights(const moe_config* cfg, const void* w, void* wt,
                                       void* stream) {
  Dims D;
  moe_status st = check_train_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  K2_PTR(w, "w");
  K2_PTR(wt, "wt");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t d = (size_t)D.d, I = (size_t)D.I, es = 3 * I * d;
  const uint16_t* src = static_cast<const uint16_t*>(w);
  uint16_t* dst = static_cast<uint16_t*>(wt);
  // expert g: down^T [I, d] at g * 3Id, [gate; up]^T [d, 2I] at g * 3Id + Id,
  // both K-blocked
  K2_HIP(k2::launch_transpose_w(D.G, (int)d, (int)I, src + 2 * I * d, es, (int)I, dst, es, 0,
                                s));
  K2_HIP(k2::launch_transpose_w(D.G, (int)I, (int)d, src, es, (int)d, dst + I * d, es, 0, s));
  K2_HIP(k2::launch_transpose_w(D.G, (int)I, (int)d, src + I * d, es, (int)d, dst + I * d, es,
                                (int)I, s));
  return MOE_OK;
}

moe_status moe_train_saved_bytes(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims D;
  moe_status st = check_train_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  K2_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = train_saved(D).total;
  return MOE_OK;
}

moe_status moe_train_workspace_bytes(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims D;
  moe_status st = check_train_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  K2_REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = train_layout(D).total;
  return MOE_OK;
}

moe_status moe_train_forward(const moe_config* cfg, int64_t T, const void* x, const void* norm_w,
                             const void* w_router, const float* bias, const void* w, void* out,
                             void* saved, void* ws, size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_train_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(x, "x");
  K2_PTR(norm_w, "norm_w");
  K2_PTR(w_router, "w_router");
  K2_PTR4(bias, "bias");
  K2_PTR(w, "w");
  K2_PTR(out, "out");
  K2_PTR(saved, "saved");
  K2_PTR(ws, "ws");
  const TrainLayout L = train_layout(D);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE,
             "workspace too small: need " + std::to_string(L.total));
  const TrainSaved v = train_saved(D);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* ids = at<int32_t>(saved, v.ids);
  float* wts = at<float>(saved, v.w);
  int32_t* offsets = at<int32_t>(saved, v.offsets);
  int32_t* row_pair = at<int32_t>(saved, v.row_pair);
  // norm + FP8 copy of h (hq, hs: the kept up-projection input), router, top-k
  if ((st = run_router(D, L.fl, ws, x, norm_w, w_router, bias, ids, wts,
                       at<float>(ws, L.gap), at<void>(saved, v.hq),
                       at<float>(saved, v.hs), s)) != MOE_OK)
    return st;
  {
    Stage stg(MOE_STAGE_TOPK, s);
    K2_HIP(k2::launch_chosen_scores((int)T, D.E, D.k, at<float>(ws, L.fl.zpart), ids,
                                    at<float>(saved, v.s), s));
  }
  if ((st = run_permute(D, L.fl, ws, ids, offsets, row_pair, at<int32_t>(saved, v.pair_row), s)) !=
      MOE_OK)
    return st;
  {
    Stage stg(MOE_STAGE_TILES, s);
    K2_HIP(k2::launch_build_tiles(D.E, D.S, (int)T, D.k, 128, (int)mtile_bound(D, 128), offsets,
                                  at<int32_t>(ws, L.mt_start), at<int32_t>(ws, L.tile_group), s));
  }
  const size_t d = (size_t)D.d, I = (size_t)D.I;
  const uint16_t* W = static_cast<const uint16_t*>(w);
  k2::TrainGemmArgs a = train_rows_args(D, L, ws, offsets, row_pair);
  a.topk_w = wts;
  a.guq = at<uint8_t>(saved, v.guq);
  a.gus = at<float>(saved, v.gus);
  a.abf = at<uint16_t>(ws, L.abf);
  a.rows = at<float>(ws, L.rows);
  a.shared_out = at<float>(ws, L.shared);
  a.ldo = D.d;
  {
    Stage stg(MOE_STAGE_TRAIN_FWD, s);
    // gate/up: A = gate (A2 = up) of each expert, B = h rows by token
    a.A = W;
    a.A2 = W + I * d;
    a.a_stride = 3 * I * d;
    a.lda = D.d;
    a.B = at<uint16_t>(ws, L.fl.hbuf);
    a.ldb = D.d;
    a.K = D.d;
    a.NC = D.I / 128;
    K2_HIP(k2::launch_train_gemm(k2::TM_FWD_GU, a, train_grid(D, a.NC), s));
    // down: A = down [d, I], B = a rows
    a.A = W + 2 * I * d;
    a.A2 = nullptr;
    a.lda = D.I;
    a.B = a.abf;
    a.ldb = D.I;
    a.K = D.I;
    a.NC = D.d / 256;
    K2_HIP(k2::launch_train_gemm(k2::TM_FWD_DOWN, a, train_grid(D, a.NC), s));
  }
  Stage stg(MOE_STAGE_COMBINE, s);
  K2_HIP(k2::launch_combine(true, false, (int)T, D.d, D.k, a.rows, at<int32_t>(saved, v.pair_row),
                            wts, 0, D.S ? a.shared_out : nullptr, x, out, s));
  return MOE_OK;
}

moe_status moe_train_backward(const moe_config* cfg, int64_t T, const void* dout, const void* x,
                              const void* norm_w, const void* w_router, const void* w,
                              const void* wt, const void* saved, float* dx, float* d_norm_w,
                              float* d_w_router, float* d_w, float* dh_rows, float* dw, void* ws,
                              size_t ws_bytes, void* stream) {
  Dims D;
  moe_status st = check_train_cfg(cfg, &D);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(T, &D)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  K2_PTR(dout, "dout");
  K2_PTR(x, "x");
  K2_PTR(norm_w, "norm_w");
  K2_PTR(w_router, "w_router");
  K2_PTR(w, "w");
  K2_PTR(wt, "wt");
  K2_PTR(saved, "saved");
  K2_PTR(dx, "dx");
  K2_PTR(d_norm_w, "d_norm_w");
  K2_PTR(d_w_router, "d_w_router");
  K2_PTR(d_w, "d_w");
  K2_OPT_PTR(dh_rows, "dh_rows");
  K2_OPT_PTR4(dw, "dw");
  K2_PTR(ws, "ws");
  const TrainLayout L = train_layout(D);
  K2_REQUIRE(ws_bytes >= L.total, MOE_ERR_WORKSPACE,
             "workspace too small: need " + std::to_string(L.total));
  const TrainSaved v = train_saved(D);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* offsets = at<const int32_t>(const_cast<void*>(saved), v.offsets);
  const int32_t* row_pair = at<const int32_t>(const_cast<void*>(saved), v.row_pair);
  const int32_t* pair_row = at<const int32_t>(const_cast<void*>(saved), v.pair_row);
  const float* wts = at<const float>(const_cast<void*>(saved), v.w);
  void* sv = const_cast<void*>(saved);
  const size_t d = (size_t)D.d, I = (size_t)D.I, P = (size_t)D.P;
  const int64_t ldt = train_ldt(D);
  const uint16_t* WT = static_cast<const uint16_t*>(wt);
  float* rows = dh_rows ? dh_rows : at<float>(ws, L.rows);
  float* shared = dh_rows ? dh_rows + P * d : at<float>(ws, L.shared);
  {
    Stage stg(MOE_STAGE_TILES, s);
    K2_HIP(k2::launch_build_tiles(D.E, D.S, (int)T, D.k, 128, (int)mtile_bound(D, 128), offsets,
                                  at<int32_t>(ws, L.mt_start), at<int32_t>(ws, L.tile_group), s));
  }
  k2::TrainGemmArgs a = train_rows_args(D, L, ws, offsets, row_pair);
  a.topk_w = wts;
  a.guq = at<uint8_t>(sv, v.guq);
  a.gus = at<float>(sv, v.gus);
  a.abf = at<uint16_t>(ws, L.abf);
  a.dgu = at<uint16_t>(ws, L.dgu);
  a.dwp = at<float>(ws, L.dwp);
  a.rows = rows;
  a.shared_out = shared;
  a.ldo = D.d;
  {
    Stage stg(MOE_STAGE_TRAIN_DGRAD, s);
    // down: da_raw = W_down^T dy (A = down^T [I, d]), epilogue: a~, dw, dg, du
    a.A = WT;
    a.a_stride = 3 * I * d;
    a.lda = 32 * D.I;   // K-blocked: 32 K of all I rows per block
    a.B = static_cast<const uint16_t*>(dout);
    a.ldb = D.d;
    a.K = D.d;
    a.NC = D.I / 256;
    K2_HIP(k2::launch_train_gemm(k2::TM_BWD_DOWN, a, train_grid(D, a.NC), s));
  }
  // The weight gradients need only the down dgrad's outputs (a~, dg, du) and
  // the saved state.  The side stream forms their transposed operands and
  // dW_gate, dW_up while `stream` runs the gate/up dgrad and the router
  // backward and then dW_down (the gate/up dgrad reads weights, the weight
  // gradients mostly write; this split gives the two streams about equal
  // work); joined before returning.
  SideStream side;
  if ((st = side_stream_of_current_device(&side)) != MOE_OK) return st;
  K2_HIP(hipEventRecord(side.fork, s));
  K2_HIP(hipStreamWaitEvent(side.s2, side.fork, 0));
  if ((st = train_wgrad_transposes(D, L, T, ws, sv, v, offsets, row_pair, wts, dout, a.abf,
                                   a.dgu, side.s2)) != MOE_OK)
    return st;
  K2_HIP(hipEventRecord(side.mid, side.s2));
  if ((st = train_wgrad_gemm(D, L, ws, false, d_w, side.s2)) != MOE_OK) return st;
  K2_HIP(hipEventRecord(side.join, side.s2));
  {
    Stage stg(MOE_STAGE_TRAIN_DGRAD, s);
    // gate/up: dh_row = [W_gate; W_up]^T [dg; du] (A = [gate; up]^T [d, 2I])
    a.A = WT + I * d;
    a.lda = 32 * D.d;   // K-blocked: 32 K of all d rows per block
    a.B = a.dgu;
    a.ldb = 2 * D.I;
    a.K = 2 * D.I;
    a.NC = D.d / 256;
    K2_HIP(k2::launch_train_gemm(k2::TM_BWD_GU, a, train_grid(D, a.NC), s));
  }
  float* dh = at<float>(ws, L.dh);
  float* dz = at<float>(ws, L.dz);
  float* dht = at<float>(ws, L.dht);
  {
    Stage stg(MOE_STAGE_TRAIN_OTHER, s);
    K2_HIP(k2::launch_combine(false, true, (int)T, D.d, D.k, rows, pair_row, wts, 0,
                              D.S ? shared : nullptr, nullptr, dh, s));
    k2::RouterBwdArgs r{};
    r.T = (int)T;
    r.d = D.d;
    r.k = D.k;
    r.E = D.E;
    r.P = (int)D.P;
    r.nchunk = D.I / 256;
    r.renorm = D.renorm;
    r.scaling = D.scaling;
    r.eps = D.eps;
    r.dwp = a.dwp;
    r.pair_row = pair_row;
    r.ids = at<const int32_t>(sv, v.ids);
    r.s = at<const float>(sv, v.s);
    r.dh = dh;
    r.w_router = static_cast<const uint16_t*>(w_router);
    r.x = static_cast<const uint16_t*>(x);
    r.norm_w = static_cast<const uint16_t*>(norm_w);
    r.dout = static_cast<const uint16_t*>(dout);
    r.dz = dz;
    r.dw_out = dw;
    r.dh_total = dht;
    r.dx = dx;
    K2_HIP(k2::launch_router_norm_bwd(r, s));
    K2_HIP(k2::launch_col_sum((int)T, D.d, dht, at<double>(ws, L.colsum), d_norm_w, s));
    K2_HIP(k2::launch_router_wgrad(D.E, D.d, D.k, (int)D.P, offsets, row_pair, dz,
                                   at<const uint8_t>(sv, v.hq), at<const float>(sv, v.hs),
                                   d_w_router, s));
  }
  // dW_down, once the side stream's transposes are done
  K2_HIP(hipStreamWaitEvent(s, side.mid, 0));
  if ((st = train_wgrad_gemm(D, L, ws, true, d_w, s)) != MOE_OK) return st;
  K2_HIP(hipStreamWaitEvent(s, side.join, 0));
  return MOE_OK;
}

}  // extern "C"
