// Internal launchers of the K2 MoE kernels (host side).  Every launcher
// enqueues on `s` and returns hipGetLastError() of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace k2 {

// the thread-local text moe_last_error() returns
std::string& error_text();
// per-stage HIP-event timing (moe_profile_enable): a stage's launches are
// bracketed by profile_begin / profile_end on their stream
void* profile_begin(int stage, hipStream_t s);
void profile_end(void* handle);
struct ProfileScope {
  void* h;
  ProfileScope(int stage, hipStream_t s) : h(profile_begin(stage, s)) {}
  ~ProfileScope() { profile_end(h); }
};

// ---- norm + quant + router (norm_router.hip)
hipError_t launch_norm_quant(bool fp8, int T, int d, float eps, const void* x, const void* gamma,
                             void* hbuf, void* xq, float* xs, hipStream_t s);
hipError_t launch_router_gemm_bf16(int T, int d, int E, int ksplit, const uint16_t* h,
                                   const uint16_t* wr, float* zpart, hipStream_t s);
hipError_t launch_router_gemm_f32(int T, int d, int E, const float* h, const float* wr,
                                  float* zpart, hipStream_t s);
hipError_t launch_topk(int T, int E, int k, int ksplit, float* zpart, const float* bias,
                       float scaling, int renorm, int32_t* ids, float* w, float* gap,
                       hipStream_t s);
hipError_t launch_dense_route(int T, float scaling, int32_t* ids, float* w, float* gap,
                              hipStream_t s);

// ---- permutation (permute.hip)
int perm_chunk_tokens(int E);
// GEMM m-tile table wanted together with the permutation (see launch_build_tiles)
struct TileReq {
  int bm, max_tiles, n_shared;
  int32_t* mt_start;
  int32_t* tile_group;
};
// With tiles non-null, *tiles_built says whether the table was built too (it
// is when all tokens fit one chunk); otherwise launch_build_tiles builds it.
hipError_t launch_permute(int T, int E, int k, const int32_t* ids, int32_t* chunk_counts,
                          int32_t* chunk_base, int32_t* offsets, int32_t* row_pair,
                          int32_t* pair_row, hipStream_t s, const TileReq* tiles = nullptr,
                          bool* tiles_built = nullptr);
hipError_t launch_build_tiles(int E, int n_shared, int T, int k, int bm, int max_tiles,
                              const int32_t* offsets, int32_t* mt_start, int32_t* tile_group,
                              hipStream_t s);

// ---- grouped FP8 GEMMs (gemm_fp8.hip)
struct GemmArgs {
  const uint8_t* wpk;       // packed codes of expert 0 for this matrix kind
  size_t expert_stride;     // bytes between experts' packed codes
  const float* wscale;      // packed scales of expert 0 for this matrix kind
  size_t wscale_stride;     // floats between experts' scales
  const uint8_t* act;       // activation codes: xq [T, d] or a_q [P+T, I]
  const float* act_s;       // activation scales [rows, K/128]
  int act_ld;               // bytes per activation row (= K)
  int nkb;                  // K / 128
  const int32_t* offsets;   // expert_offsets [E+1]
  const int32_t* row_pair;  // [P]
  const int32_t* mt_start;  // [G+1] prefix of m-tiles per group
  const int32_t* tile_group;  // [mt_start[G]] group of each m-tile
  int E, G, T, k, P, NC;    // NC: 256-row weight chunks per expert
  // gate/up outputs
  uint8_t* aq;              // [P+T, I]
  float* as;                // [P+T, I/128]
  int I;
  // down outputs
  float* rows;              // [P, d]
  float* shared_out;        // [T, d]
  const float* topk_w;      // [P] pair weights, used when weighted
  int weighted;
  int d;
  // down form, one group of token rows, one K slice: if out_bf16 is set, each
  // row is written as bf16(res + row) to out_bf16 [T, d] instead of to rows
  const uint16_t* res;      // [T, d] bf16
  uint16_t* out_bf16;       // [T, d] bf16
};
hipError_t launch_gemm_fp8(bool gateup, int tt, const GemmArgs& a, int grid, hipStream_t s);

// ---- fp32 experts (gemm_f32.hip)
hipError_t launch_experts_f32(int T, int d, int I, int E, int k, int n_shared, const float* h,
                              const int32_t* offsets, const int32_t* row_pair,
                              const float* packed, size_t expert_floats, float* abuf,
                              float* rows, float* shared_out, const float* topk_w,
                              int weighted, hipStream_t s);

// ---- combine and packing (combine_pack.hip)
hipError_t launch_combine(bool x_bf16, bool out_f32, int T, int d, int k, const float* rows,
                          const int32_t* pair_row, const float* topk_w, int weighted,
                          const float* shared_out, const void* residual, void* out,
                          hipStream_t s);
hipError_t launch_pack_fp8(int d, int I, const uint8_t* wg, const uint8_t* wu,
                           const uint8_t* wd, const float* sg, const float* su,
                           const float* sd, uint8_t* dst_codes, float* dst_gu_scales,
                           float* dst_d_scales, hipStream_t s);

// ---- routing bias update (balance.hip)
hipError_t launch_expert_load(int64_t n, int E, const int32_t* ids, int32_t* counts,
                              hipStream_t s);
hipError_t launch_bias_update(int E, const int32_t* counts, float speed, float* bias,
                              hipStream_t s);

}  // namespace k2
