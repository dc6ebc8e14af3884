// Internal launchers of the MLA attention kernels (host side).  Every launcher
// enqueues on `s` and returns hipGetLastError() of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k2_launch.h"

namespace k2 {

// packing of one projection matrix (or two stacked) into the grouped GEMM's
// down-form layout, zero rows up to n_pad; scales padded with 1.0
hipError_t launch_pack_rows(int n_pad, int K, const uint8_t* src0, int n0, const uint8_t* src1,
                            int n1, const float* s0, const float* s1, uint8_t* dst_codes,
                            float* dst_scales, hipStream_t s);
// tables of one group of T rows for the grouped GEMM
hipError_t launch_dense_tiles(int T, int bm, int32_t* offsets, int32_t* mt_start,
                              int32_t* tile_group, hipStream_t s);
// the dense FP8 GEMM rows[k, T, d] = partial sums of slice k (a.rows, a.d = padded N);
// tt = 1, 2 or 4 (16-, 32-, 64-row m-tiles)
hipError_t launch_gemm_dense(int tt, int nsplit, const GemmArgs& a, int grid, hipStream_t s);
// sum of K slices, optionally + bf16 residual and rounding to bf16
hipError_t launch_slice_sum(int T, int ncol, int ld, int nsplit, const float* part,
                            const uint16_t* residual, void* out, int out_ld, hipStream_t s);
// qkv: nsplit K-slice partial sums [nsplit, T, qkv_ld] of the [q_a; kv_a] projection;
// rot (optional) [T, 32, 2]: cosine and sine of each token's rotary angles
hipError_t launch_mla_latent(int T, int nsplit, int q_lora, int qkv_ld, float eps,
                             const float* qkv, const uint16_t* g_qa, const uint16_t* g_kva,
                             const double* inv_freq, const int32_t* cached_len, int n_new,
                             int max_len, uint8_t* qa_q, float* qa_s, uint8_t* c_codes,
                             float* c_scales, uint16_t* c_rope, double* rot, hipStream_t s);
// bf16 copies of the key-value up-projection's codes: ukt [H][512][128] (key
// rows transposed), uv [H][128][512] (value rows), uk [H][128][512] (key rows)
hipError_t launch_mla_pack_ukv(int H, const uint8_t* w_kvb, uint16_t* ukt, uint16_t* uv,
                              uint16_t* uk, hipStream_t s);
// q: nsplit K-slice partial sums [nsplit, T, H * 192] of the q_b projection;
// qcat [T, H, 2, 576]: the absorbed queries (softmax scale folded in) as their
// bf16 high parts, then the bf16 roundings of the remainders
hipError_t launch_mla_qabsorb(int T, int H, int nsplit, float smscale, const float* q,
                              const uint16_t* ukt,
                              const float* s_kvb, const double* inv_freq,
                              const int32_t* cached_len, int n_new, int max_len, uint16_t* qcat,
                              hipStream_t s);
// work items per position split of the attention kernel, and its mode:
// mode 0 (one new token per sequence and heads a multiple of min(heads, 64)):
// (token, group of hw = min(heads, 64) heads); mode 1: (sequence, 8 new
// tokens, 8 heads)
inline int mla_attn_items(int T, int H, int n_seq, int n_new, int* mode, int* hw) {
  const int w = H < 64 ? H : 64;
  if (n_new == 1 && H % w == 0) {
    *mode = 0;
    *hw = w;
    return T * (H / w);
  }
  *mode = 1;
  *hw = 8;
  return n_seq * ((n_new + 7) / 8) * (H / 8);
}
hipError_t launch_mla_attn(int T, int H, int n_seq, int n_new, int max_len, int nsplit,
                           int chunk, const uint8_t* c_codes, const float* c_scales,
                           const uint16_t* c_rope, const uint16_t* qcat,
                           const int32_t* cached_len, float* part_o, float* part_ml,
                           hipStream_t s);
// Per-head attention for prompt-sized batches (mla_mha.hip): the keys and
// values of every visible position and head are formed from the cache into
// kv (mla_mha_kv_bytes, nblk blocks of 32 positions per (sequence, head)),
// then attended; rot: the new tokens' rotations from launch_mla_latent; writes
// o_q / o_s (and attn if not null) as launch_mla_vup does.
int mla_mha_nblk(int max_len);
size_t mla_mha_kv_bytes(int n_seq, int H, int max_len);
hipError_t launch_mla_mha(int T, int H, int n_seq, int n_new, int max_len, int nsplit,
                          float smscale, const float* q, const double* rot,
                          const int32_t* cached_len, const uint8_t* c_codes,
                          const float* c_scales, const uint16_t* c_rope, const uint16_t* uk,
                          const uint16_t* uv, const float* s_kvb, uint16_t* kv, uint8_t* o_q,
                          float* o_s, float* attn, hipStream_t s);
hipError_t launch_mla_vup(int T, int H, int nsplit, const float* part_o, const float* part_ml,
                          const uint16_t* uv, const float* s_kvb, uint8_t* o_q, float* o_s,
                          float* attn, hipStream_t s);

}  // namespace k2
