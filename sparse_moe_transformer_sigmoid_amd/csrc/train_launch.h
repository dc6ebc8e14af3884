// Internal launchers of the training-step kernels (train.hip).  Every
// launcher enqueues on `s` and returns hipGetLastError() of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace k2 {

// products of the bf16 grouped GEMM kernel
enum { TM_FWD_GU = 0, TM_FWD_DOWN = 1, TM_BWD_DOWN = 2, TM_BWD_GU = 3, TM_WGRAD = 4 };

// M rows (output features) of a weight-gradient tile: TrainGemmArgs::MT of a
// TM_WGRAD launch counts tiles of this height
constexpr int WGRAD_M = 256;

struct TrainGemmArgs {
  // groups and rows (row-tiled products): routed rows in expert order, then
  // the shared expert's T rows at P .. P + T
  const int32_t* offsets;     // [E+1]
  const int32_t* row_pair;    // [P] routed row -> (token, slot) pair
  const int32_t* mt_start;    // [G+1] 128-row tiles per group (prefix)
  const int32_t* tile_group;  // group of each tile
  int E, G, T, P, k;
  int NC;                     // 256-row M chunks per group (row-tiled products)
  int K;                      // reduction length (row-tiled products)
  // A: 256-row M chunks streamed into registers (bf16, K contiguous)
  const uint16_t* A;          // group 0's matrix (forward gate/up: the gate matrix)
  const uint16_t* A2;         // forward gate/up: the up matrix
  size_t a_stride;            // elements between groups' matrices
  int lda;                    // row stride; dgrad and wgrad: elements per 32-column K block
  // B: 128 rows staged through LDS (bf16, K contiguous)
  const uint16_t* B;
  int ldb;                    // row stride; wgrad: elements per 32-column K block
  // wgrad: padded column offsets of the groups in the transposed operands,
  // 256-row M tiles and 128-column N tiles per group, gradient output
  const int32_t* pad_off;     // [G+1]
  int MT, NT;
  float* out;
  size_t out_stride;          // floats between groups' gradients
  int ldo;                    // floats per output row (also the fp32 row stride below)
  // epilogue data
  int I;
  const float* topk_w;        // [P] routing weight of each pair
  uint8_t* guq;               // [R, 2I] FP8 copies of g (first I) and u
  float* gus;                 // [R, 2I/128] their scales
  uint16_t* abf;              // [R, I] bf16 a (forward) or a~ (backward)
  uint16_t* dgu;              // [R, 2I] bf16 dg (first I) and du
  float* dwp;                 // [R, NC] partial routing-weight gradients
  float* rows;                // [P, ldo] fp32 routed rows
  float* shared_out;          // [T, ldo] fp32 shared rows
};
hipError_t launch_train_gemm(int mode, const TrainGemmArgs& a, int grid, hipStream_t s);

struct TransposeArgs {
  const uint16_t* src;        // mode 0: [R, C]; mode 1: dy [T, C]
  const uint8_t* codes;       // mode 2: FP8 h [T, C]
  const float* scales;        // mode 2: [T, C/128]
  const int32_t* offsets;     // [E+1]
  const int32_t* row_pair;    // [P]
  const float* topk_w;        // [P] (mode 1)
  const int32_t* pad_off;     // [G+1]
  int E, G, T, P, k, C;
  uint16_t* dst;              // ldt / 32 K blocks of [C][32]
  int ldt;
};
hipError_t launch_pad_offsets(int E, int G, int T, int P, const int32_t* offsets,
                              int32_t* pad_off, hipStream_t s);
hipError_t launch_transpose_pad(int src_mode, const TransposeArgs& a, int padded_cols,
                                hipStream_t s);
// n [R][C] bf16 matrices -> K-blocked transposes: element (c, k = dst_col0 + r)
// at ((k / 32) * C + c) * 32 + k % 32
hipError_t launch_transpose_w(int n, int R, int C, const uint16_t* src, size_t src_stride,
                              int src_ld, uint16_t* dst, size_t dst_stride, int dst_col0,
                              hipStream_t s);

hipError_t launch_chosen_scores(int T, int E, int k, const float* z, const int32_t* ids,
                                float* sc, hipStream_t s);

struct RouterBwdArgs {
  int T, d, k, E, P, nchunk, renorm;
  float scaling, eps;
  const float* dwp;           // [R, nchunk]
  const int32_t* pair_row;    // [P]
  const int32_t* ids;         // [T, k]
  const float* s;             // [T, k]
  const float* dh;            // [T, d] from the experts
  const uint16_t* w_router;   // [E, d]
  const uint16_t* x;          // [T, d]
  const uint16_t* norm_w;     // [d]
  const uint16_t* dout;       // [T, d]
  float* dz;                  // [T, k]
  float* dw_out;              // [T, k] (optional)
  float* dh_total;            // [T, d] scratch; ends holding each token's dgamma term
  float* dx;                  // [T, d]
};
hipError_t launch_router_norm_bwd(const RouterBwdArgs& a, hipStream_t s);
size_t col_sum_scratch_bytes(int T, int d);
hipError_t launch_col_sum(int T, int d, const float* in, double* scratch, float* out,
                          hipStream_t s);
hipError_t launch_router_wgrad(int E, int d, int k, int P, const int32_t* offsets,
                               const int32_t* row_pair, const float* dz, const uint8_t* hq,
                               const float* hs, float* dwr, hipStream_t s);

}  // namespace k2
