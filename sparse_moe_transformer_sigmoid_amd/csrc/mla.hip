// Kimi K2 multi-head latent attention (MLA) on gfx950: the kernels between the
// FP8 projections.
//
// Shape ("Kimi K2 · Architecture", Fact sheet and config.json; "Kimi-K2-Base",
// Attention): 64 heads; a 1,536-wide query latent and a 512-wide key-value
// latent, each RMS-normalised before its up-projection; per head 128
// query/key features without position, 64 rotary ones (one rotary key shared
// by the heads) and 128 value features; softmax scale (0.1 ln 32 + 1)^2 /
// sqrt(192); causal; positions numbered from the cached length.
//
// Decode and small chunks attend in the absorbed form over the latent cache
// (below); prompt-sized batches use the per-head form of mla_mha.hip.  With W_uk,
// W_uv the key and value rows of head h's key-value up-projection and c_j the
// cached latent of position j:
//   q_nope . (W_uk c_j) = (W_uk^T q_nope) . c_j,
//   sum_j p_j (W_uv c_j) = W_uv (sum_j p_j c_j),
// so a query becomes q_lat = [W_uk^T q_nope, rope(q_pe)] (576 wide), every
// head scores against the same cache rows [c_j, k_rope_j], and the value
// up-projection is applied once to the weighted latent sum.  The cache holds
// c_j as the e4m3 codes and 1x128 scales the FP8 key-value up-projection
// reads (656 bytes per position with the bf16 rotary key).
#include <math.h>

#include "k2_common.h"
#include "mla_common.h"
#include "mla_launch.h"

namespace k2 {

namespace {

constexpr int PT = 32;            // cache positions per attention step
constexpr int CT_LD = DL + 8;     // bf16 stride of a row-major cache latent in LDS
// bf16 stride of a transposed latent row in LDS: 18 dwords, so the four
// 16-row chunks a fill wave writes in one instruction fall on two bank halves
// and the 16 rows a compute wave reads on 16 distinct even banks
constexpr int TR_LD = PT + 4;

// ------------------------------------------------------------------ packing
// [n0 rows of src0; n1 rows of src1; zero rows] x K codes -> the grouped GEMM's
// down-form fragment order (256-row chunks, four 64-row waves, K blocks, 16-row
// tiles, lane halves), as the expert down projections are packed.
__global__ __launch_bounds__(256) void pack_rows_kernel(int n_pad, int K, const uint8_t* src0,
                                                        int n0, const uint8_t* src1, int n1,
                                                        uint8_t* __restrict__ dst) {
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  if (q >= (long)n_pad * K / 16) return;
  const int lane = q & 63, p = (q >> 6) & 1, rt = (q >> 7) & 3;
  long rest = q >> 9;
  const int nkb = K / QBLK;
  const int kb = (int)(rest % nkb);
  rest /= nkb;
  const int w = (int)(rest & 3), j = (int)(rest >> 2);
  const int row = j * 256 + 64 * w + 16 * rt + (lane & 15);
  const int col = kb * 128 + (lane >> 4) * 32 + p * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < n0)
    v = *reinterpret_cast<const uint4*>(src0 + (size_t)row * K + col);
  else if (row < n0 + n1)
    v = *reinterpret_cast<const uint4*>(src1 + (size_t)(row - n0) * K + col);
  reinterpret_cast<uint4*>(dst)[q] = v;
}

// block scales [ceil(n0/128) of s0; ceil(n1/128) of s1; 1.0 padding] x K/128
__global__ void pack_row_scales_kernel(int nb_pad, int kb, const float* s0, int nb0,
                                       const float* s1, int nb1, float* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nb_pad * kb) return;
  const int rb = i / kb, c = i % kb;
  float v = 1.f;
  if (rb < nb0) v = s0[rb * kb + c];
  else if (rb < nb0 + nb1) v = s1[(rb - nb0) * kb + c];
  dst[i] = v;
}

// the grouped GEMM's tables for one group of T rows (offsets, m-tile prefix,
// m-tile -> group)
__global__ void dense_tiles_kernel(int T, int bm, int32_t* offsets, int32_t* mt_start,
                                   int32_t* tile_group) {
  const int n = (T + bm - 1) / bm;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
    mt_start[0] = 0;
    mt_start[1] = n;
  }
  if (i < n) tile_group[i] = 0;
}

// out[t, c] = sum over s of part[s, t, c] (ascending s), c < ncol of rows of
// width ld; then + residual and one rounding to bf16 (res != null), or fp32.
__global__ __launch_bounds__(256) void slice_sum_kernel(int T, int ncol, int ld, int nsplit,
                                                        const float* __restrict__ part,
                                                        const uint16_t* __restrict__ res,
                                                        void* __restrict__ out, int out_ld) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * (ncol / 4)) return;
  const int t = (int)(i / (ncol / 4)), c = 4 * (int)(i % (ncol / 4));
  float4 a = *reinterpret_cast<const float4*>(part + (size_t)t * ld + c);
  for (int s = 1; s < nsplit; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(part + ((size_t)s * T + t) * ld + c);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  if (res) {
    const uint2 xr = *reinterpret_cast<const uint2*>(res + (size_t)t * out_ld + c);
    const uint32_t o0 = f32_to_bf16_rne(bf16_to_f32(xr.x & 0xFFFFu) + a.x) |
                        (f32_to_bf16_rne(bf16_to_f32(xr.x >> 16) + a.y) << 16);
    const uint32_t o1 = f32_to_bf16_rne(bf16_to_f32(xr.y & 0xFFFFu) + a.z) |
                        (f32_to_bf16_rne(bf16_to_f32(xr.y >> 16) + a.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * out_ld + c) =
        make_uint2(o0, o1);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * out_ld + c) = a;
  }
}

// ------------------------------------------------------- latents and cache

// Per token: RMSNorm of the query latent -> bf16 -> 1x128 codes (the input of
// the query up-projection); RMSNorm of the key-value latent -> bf16 -> 1x128
// codes and scales into the cache; the positional key rotated and rounded to
// bf16 into the cache.  qkv row: [q_a (q_lora), kv_a latent (512), k_pe (64)].
// Norms as in the input RMSNorm: mean of squares formed in fp64, rounded to
// fp32, r = 1/sqrt(ms + eps), h = bf16((v r) g).
constexpr int MAX_QKV = 8192 + DL + DR;   // longest [q_a; kv_a] row (q_lora <= 8192)

// qkv: the [q_a; kv_a] projection as nsplit K-slice partial sums [nsplit, T,
// qkv_ld], added in slice order (the order of launch_slice_sum).
__global__ __launch_bounds__(256) void mla_latent_kernel(
    int T, int nsplit, int q_lora, int qkv_ld, float eps, const float* __restrict__ qkv,
    const uint16_t* __restrict__ g_qa, const uint16_t* __restrict__ g_kva,
    const double* __restrict__ inv_freq, const int32_t* __restrict__ cached_len, int n_new,
    int max_len, uint8_t* __restrict__ qa_q, float* __restrict__ qa_s,
    uint8_t* __restrict__ c_codes, float* __restrict__ c_scales, uint16_t* __restrict__ c_rope,
    double* __restrict__ rot) {
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int seq;
  const int pos = token_pos(cached_len, t, n_new, max_len, &seq);
  const size_t cidx = (size_t)seq * max_len + pos;
  __shared__ double red[2][4];
  __shared__ float rowbuf[MAX_QKV];
  const int nrow = q_lora + DL + DR;
  for (int i = tid; i < nrow; i += 256) {
    float a = qkv[(size_t)t * qkv_ld + i];
    for (int s = 1; s < nsplit; ++s) a += qkv[((size_t)s * T + t) * qkv_ld + i];
    rowbuf[i] = a;
  }
  __syncthreads();
  const float* row = rowbuf;
  // sums of squares: query latent (q_lora values) and key-value latent (512)
  double sq = 0.0, sc = 0.0;
  for (int i = tid; i < q_lora; i += 256) sq += (double)row[i] * (double)row[i];
  for (int i = tid; i < DL; i += 256) sc += (double)row[q_lora + i] * (double)row[q_lora + i];
  sq = wave_sum(sq);
  sc = wave_sum(sc);
  if (lane == 0) {
    red[0][wave] = sq;
    red[1][wave] = sc;
  }
  __syncthreads();
  const float msq = (float)((red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (double)q_lora);
  const float msc = (float)((red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (double)DL);
  const float rq = 1.0f / sqrtf(msq + eps), rc = 1.0f / sqrtf(msc + eps);
  // a wave normalises and quantises 128-value blocks, two values per lane
  auto quant_block = [&](const float* src, const uint16_t* g, float r, uint8_t* codes,
                         float* scale) {
    const int i = 2 * lane;
    const float h0 = bf16_to_f32(f32_to_bf16_rne((src[i] * r) * bf16_to_f32(g[i])));
    const float h1 = bf16_to_f32(f32_to_bf16_rne((src[i + 1] * r) * bf16_to_f32(g[i + 1])));
    float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float s = fp8_scale(amax);
    const uint32_t q = cvt4_e4m3(clamp_fp8(h0 / s), clamp_fp8(h1 / s), 0.f, 0.f);
    *reinterpret_cast<uint16_t*>(codes + i) = (uint16_t)(q & 0xFFFFu);
    if (lane == 0) *scale = s;
  };
  const int nqb = q_lora / QBLK;
  for (int b = wave; b < nqb; b += 4)
    quant_block(row + b * QBLK, g_qa + b * QBLK, rq, qa_q + (size_t)t * q_lora + b * QBLK,
                qa_s + (size_t)t * nqb + b);
  quant_block(row + q_lora + wave * QBLK, g_kva + wave * QBLK, rc,
              c_codes + cidx * DL + wave * QBLK, c_scales + cidx * (DL / QBLK) + wave);
  if (tid < DR / 2) {
    double sn, cs;
    sincos((double)pos * inv_freq[tid], &sn, &cs);
    float ra, rb;
    rope_apply(row[q_lora + DL + 2 * tid], row[q_lora + DL + 2 * tid + 1], cs, sn, &ra, &rb);
    c_rope[cidx * DR + 2 * tid] = bf16_bits(ra);
    c_rope[cidx * DR + 2 * tid + 1] = bf16_bits(rb);
    // the token's rotation of pair tid, for the queries of the per-head form
    if (rot) {
      rot[((size_t)t * (DR / 2) + tid) * 2] = cs;
      rot[((size_t)t * (DR / 2) + tid) * 2 + 1] = sn;
    }
  }
}

// --------------------------------------------------------- query absorption
// ------------------------------------------------------- latent attention
// Eight waves, each scoring a column block of 8 (token, head) pairs.  mode 0
// (one new token per sequence): the waves are one token's groups of 8 heads,
// so a workgroup covers min(heads, 64) heads and reads each cache position
// once for all of them; mode 1: up to eight consecutive tokens of one sequence
// with one group of 8 heads.  Waves 2i and 2i + 1 form a pair whose 16
// columns share the value sum: each wave accumulates the outputs of all 16
// columns over one half of the latent (256 features), taking the partner's
// probabilities through LDS, so it holds 64 accumulator registers, not 128.  The cache positions [lo, hi) of the work item's split are
// visited in steps of 32.  The cache bytes of a step (latent codes, rotary
// keys, scales) are copied straight from global memory into one of NS LDS
// stages (global_load_lds, no staging registers), NS - 1 steps ahead of the
// compute.  Per step every wave first converts its share of the step's codes
// into exact bf16 values (every e4m3 value is one), twice -- row-major
// [pos][512] (the A operand of the scores) and transposed [latent][pos] (the
// A operand of the value sum) -- and then computes; the rotary keys and the
// scales are read from their stage as they arrived.
//
// Sums to fp32 precision: the 16 MFMA columns are 8 heads x {hi, lo}, the
// bf16 high part of a value and the bf16 rounding of its remainder, so one
// MFMA gives both halves of the product and the two columns of a head add to
// it within about 2^-17 relative.  Per 128-latent block b:
//   S_b^T = C_b Q^T              (codes, query halves; lane: 4 positions x 1 column)
//   s = sum_b scale_b(pos) S_b + S_rope, the two columns of a head added
//   online softmax per head
//   O_b^T [latent, pair column] += C_b^T (p scale_b)^T as two MFMAs on one
//                                  cache fragment, the high and the low halves
//                                  of p scale_b; the lane's 8 K slots are
//                                  positions 4q..4q+3 of the first 16 and of
//                                  the second 16 (where S^T left them)
// and finally writes its running max m, sum l and O^T (head x 512) unscaled.
struct AttnArgs {
  const uint8_t* c_codes;
  const float* c_scales;
  const uint16_t* c_rope;
  const float* qcat;         // [T, H, 576] fp32, softmax scale folded in
  const int32_t* cached_len; // [S]
  float* part_o;             // [nsplit, T, H, 512]
  float* part_ml;            // [nsplit, T, H, 2]
  int T, H, n_new, max_len, nsplit, chunk, mode, items_per_split;
  int hw;                    // mode 0: heads per workgroup
};

// the value of the lane 8 apart in the same 16-lane row (a row rotated by 8)
__device__ __forceinline__ float xor8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), 0x128 /* row_ror:8 */, 0xF, 0xF, false));
}

constexpr int CT_ELEMS = PT * CT_LD, TR_ELEMS = DL * TR_LD;
constexpr int HPW = 8;   // heads per wave
constexpr int AW = 8;    // waves per workgroup
constexpr int NS = 3;    // LDS stages of raw cache bytes (copies run NS - 1 steps ahead)
constexpr float LAZY_E = 5.5451774f;   // 8 ln 2: margin before a head's reference maximum moves

__global__ __launch_bounds__(512, 1) void mla_attn_kernel(const AttnArgs g) {
  // raw stages: codes [pos][512] with the 16-byte chunk c of position p at
  // chunk slot c ^ ((p / 2) % 16); rotary keys [pos][64] bf16 with chunk c at
  // slot c ^ ((p / 2) % 8) (both so that 16 consecutive positions read at one
  // chunk fall on distinct banks); scales [block][pos]
  __shared__ __attribute__((aligned(16))) uint8_t cr[NS][PT * DL];
  __shared__ __attribute__((aligned(16))) uint16_t crope[NS][PT * DR];
  __shared__ __attribute__((aligned(16))) float csc[NS][DL / QBLK][PT];
  __shared__ __attribute__((aligned(16))) uint16_t ct[CT_ELEMS];   // row-major bf16 latents
  __shared__ __attribute__((aligned(16))) uint16_t tr[TR_ELEMS];   // transposed bf16 latents
  __shared__ float xbuf[AW][9][64];   // a wave's probabilities (8) and rescale factor per lane
  __shared__ int kv_sh[AW], tok_sh[AW], head_sh[AW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, l16 = lane & 15;
  const bool lo_col = l16 >= HPW;           // this lane's column holds the low halves
  const float lo_f = lo_col ? 1.f : 0.f;
  const int item = blockIdx.x % g.items_per_split, split = blockIdx.x / g.items_per_split;
  // the wave's token and first head (every wave of a workgroup is on one
  // sequence; waves past the token count or the head count only convert)
  int t, h0;
  bool active;
  if (g.mode == 0) {
    const int ngrp = g.H / g.hw;
    t = item / ngrp;
    h0 = (item % ngrp) * g.hw + wave * HPW;
    active = wave * HPW < g.hw;
  } else {
    const int hg_n = g.H / HPW;
    const int tb_n = (g.n_new + AW - 1) / AW;
    const int per_seq = tb_n * hg_n;
    const int s_ = item / per_seq, rem = item % per_seq;
    const int tb = rem / hg_n;
    h0 = (rem % hg_n) * HPW;
    const int ti = tb * AW + wave;
    active = ti < g.n_new;
    t = s_ * g.n_new + min(ti, g.n_new - 1);
  }
  int seq;
  const int qpos = token_pos(g.cached_len, t, g.n_new, g.max_len, &seq);
  if (lane == 0) {
    kv_sh[wave] = active ? qpos + 1 : 0;
    tok_sh[wave] = t;
    head_sh[wave] = h0;
  }
  __syncthreads();
  // the workgroup's positions: its split's range, up to its last query position
  int wg_end = 0;
#pragma unroll
  for (int w = 0; w < AW; ++w) wg_end = max(wg_end, kv_sh[w]);
  const int lo = split * g.chunk, hi = min(wg_end, lo + g.chunk);
  const int my_end = active ? qpos + 1 : 0;
  const int pm = wave & 1;   // member of the wave pair
  const int pair_end = max(kv_sh[wave & ~1], kv_sh[wave | 1]);   // 0: both members idle
  const int h = h0 + (l16 & (HPW - 1));   // this lane's head
  const size_t cbase = (size_t)seq * g.max_len;
  const uint8_t* codes_seq = g.c_codes + cbase * DL;
  const uint16_t* rope_seq = g.c_rope + cbase * DR;
  const float* sc_seq = g.c_scales + cbase * (DL / QBLK);

  // copies of the step at p0 into stage st; positions past hi copy position
  // hi - 1 (written, finite), which the mask and p = 0 leave without effect.
  // Wave w: code instructions 2w, 2w + 1 (two positions each); waves 0-3 one
  // rotary instruction (8 positions), waves 4-5 one scale instruction (two
  // blocks): 3 copies per step for waves 0-5, 2 for waves 6-7
  const int n_copies = wave < 6 ? 3 : 2;
  auto issue = [&](int st, int p0) {
    const int plast = hi - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * wave + u;
      const int pc = min(p0 + 2 * i + (lane >> 5), plast);
      const int c = (lane & 31) ^ (i & 15);
      lds_copy16(codes_seq, (uint32_t)(pc * DL + 16 * c), lds_addr(&cr[st][i * 1024]));
    }
    if (wave < 4) {
      const int p = 8 * wave + (lane >> 3);
      const int pc = min(p0 + p, plast);
      const int c = (lane & 7) ^ ((p >> 1) & 7);
      lds_copy16(rope_seq, (uint32_t)(pc * DR * 2 + 16 * c), lds_addr(&crope[st][wave * 512]));
    } else if (wave < 6) {
      const int i = wave - 4, blk = 2 * i + (lane >> 5);
      const int pc = min(p0 + (lane & 31), plast);
      lds_copy4(sc_seq, (uint32_t)((pc * (DL / QBLK) + blk) * 4), lds_addr(&csc[st][2 * i][0]));
    }
  };
  // stage st's codes -> ct, tr: thread = (16-code chunk sub, position pair pr)
  auto convert = [&](int st) {
    const int sub = tid >> 4, pr = tid & 15;
    uint32_t pk[2][8];   // bf16 pairs: codes 2k, 2k+1 of position 2 pr + j
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 cv =
          *reinterpret_cast<const uint4*>(&cr[st][(2 * pr + j) * DL + 16 * (sub ^ pr)]);
      const uint32_t w4[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pk[j][2 * k] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[k], 1.f, false));
        pk[j][2 * k + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[k], 1.f, true));
      }
      uint4* dst = reinterpret_cast<uint4*>(&ct[(2 * pr + j) * CT_LD + 16 * sub]);
      dst[0] = make_uint4(pk[j][0], pk[j][1], pk[j][2], pk[j][3]);
      dst[1] = make_uint4(pk[j][4], pk[j][5], pk[j][6], pk[j][7]);
    }
    // transposed: feature 16 sub + i, positions 2 pr and 2 pr + 1 (i is a
    // compile-time index: a per-thread index into pk would become select
    // chains over all its registers)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int w = i >> 1;
      const uint32_t v = (i & 1) ? ((pk[0][w] >> 16) | (pk[1][w] & 0xFFFF0000u))
                                 : ((pk[0][w] & 0xFFFFu) | (pk[1][w] << 16));
      *reinterpret_cast<uint32_t*>(&tr[(16 * sub + i) * TR_LD + 2 * pr]) = v;
    }
  };

  // the query of head h as B fragments, high or low halves by column (dims
  // 32 ks + 8 q4 .. + 7)
  v8bf qb[DQ / 32];
  v4f o[DL / 32];   // pair column l mod 16, latents 256 pm + 16 nt + 4 q4 + i
  float mrun = -INFINITY, lrun = 0.f;
#pragma unroll
  for (int i = 0; i < DL / 32; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};
  if (active) {
    const float* qp = g.qcat + ((size_t)t * g.H + h) * DQ + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(qp + 32 * ks);
      const float4 c = *reinterpret_cast<const float4*>(qp + 32 * ks + 4);
      const uint4 v = make_uint4(bf16_half2(a.x, a.y, lo_f), bf16_half2(a.z, a.w, lo_f),
                                 bf16_half2(c.x, c.y, lo_f), bf16_half2(c.z, c.w, lo_f));
      qb[ks] = __builtin_bit_cast(v8bf, v);
    }
  }
  // scores and online softmax of the wave's 8 heads; ps, alpha: the lane's
  // probabilities and the rescale factor of its head
  auto scores = [&](int st, int p0, float (&ps)[2][4], float& alpha) {
    // ---- scores: S^T[pos, column] for positions p0 + 16 pt + 4 q4 + i
    v4f s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int blk = 0; blk <= DL / QBLK; ++blk) {   // four latent blocks, then the rotary key
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const int p = 16 * pt + l16;
        if (blk < DL / QBLK) {
          const uint16_t* ap = &ct[p * CT_LD + 8 * q4];
#pragma unroll
          for (int ks = blk * 4; ks < blk * 4 + 4; ++ks) {
            const uint4 av = *reinterpret_cast<const uint4*>(ap + 32 * ks);
            acc = mfma_bf16(__builtin_bit_cast(v8bf, av), qb[ks], acc);
          }
        } else {
#pragma unroll
          for (int ks = DL / 32; ks < DQ / 32; ++ks) {
            const int c = 4 * (ks - DL / 32) + q4;   // rotary chunk of 8 features
            const uint4 av = *reinterpret_cast<const uint4*>(
                &crope[st][p * DR + 8 * (c ^ ((p >> 1) & 7))]);
            acc = mfma_bf16(__builtin_bit_cast(v8bf, av), qb[ks], acc);
          }
        }
        if (blk < DL / QBLK) {
          const float4 sc = *reinterpret_cast<const float4*>(&csc[st][blk][16 * pt + 4 * q4]);
          s[pt][0] = fmaf(sc.x, acc[0], s[pt][0]);
          s[pt][1] = fmaf(sc.y, acc[1], s[pt][1]);
          s[pt][2] = fmaf(sc.z, acc[2], s[pt][2]);
          s[pt][3] = fmaf(sc.w, acc[3], s[pt][3]);
        } else {
          s[pt] += acc;
        }
        // operand reads stay with their block (hoisting all 18 at once would
        // exceed the register budget)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the head's two columns (high and low query halves) add to its score
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[pt][i] += xor8(s[pt][i]);
    // causal mask and the step's maximum for head h (position p0 <= qpos is
    // visible, so the maximum is finite)
    float mx = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = p0 + 16 * pt + 4 * q4 + i;
        if (p >= my_end || p >= hi) s[pt][i] = -INFINITY;
        mx = fmaxf(mx, s[pt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // the reference maximum moves only when the step's maximum passes it by
    // more than LAZY_E, so the probabilities stay below e^LAZY_E and the
    // outputs are rarely rescaled; the merge and the final normalisation
    // use the same reference, which cancels exactly
    const float mnew = mx > mrun + LAZY_E ? mx : mrun;
    alpha = __expf(mrun - mnew);
    float lsum = 0.f;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ps[pt][i] = __expf(s[pt][i] - mnew);
        lsum += ps[pt][i];
      }
    // each lane keeps the sum over its own positions; the four lanes of a
    // column are added once, at the end
    lrun = lrun * alpha + lsum;
    mrun = mnew;
  };
  // value sum of the pair's 16 columns over latents 256 pm .. + 255: column
  // l mod 16 belongs to member (l mod 16) / 8, whose lane l holds its
  // probabilities at the same positions
  auto values = [&](int st) {
    const bool own = (l16 >> 3) == pm;
    float v[2][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j >> 2][j & 3] = xbuf[own ? wave : wave ^ 1][j][lane];
    const float a_col = xbuf[own ? wave : wave ^ 1][8][lane];
    // rescale only when some column's reference moved (alpha = 1 leaves them)
    if (__any(a_col != 1.f)) {
#pragma unroll
      for (int nt = 0; nt < DL / 32; ++nt) o[nt] *= a_col;
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int blk = 2 * pm + bb;
      // B: the 8 positions 4 q4 .. + 3 of both 16-position groups, high
      // halves (pbh) and low halves (pbl); one A fragment feeds both
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const float4 sc = *reinterpret_cast<const float4*>(&csc[st][blk][16 * pt + 4 * q4]);
        const float x0 = v[pt][0] * sc.x, x1 = v[pt][1] * sc.y;
        const float x2 = v[pt][2] * sc.z, x3 = v[pt][3] * sc.w;
        hv[2 * pt] = pack_bf16(x0, x1);
        hv[2 * pt + 1] = pack_bf16(x2, x3);
        lv[2 * pt] = bf16_half2(x0, x1, 1.f);
        lv[2 * pt + 1] = bf16_half2(x2, x3, 1.f);
      }
      const v8bf pbh = __builtin_bit_cast(v8bf, make_uint4(hv[0], hv[1], hv[2], hv[3]));
      const v8bf pbl = __builtin_bit_cast(v8bf, make_uint4(lv[0], lv[1], lv[2], lv[3]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const uint16_t* tp = &tr[(16 * (8 * blk + nt) + l16) * TR_LD + 4 * q4];
        const uint2 a0 = *reinterpret_cast<const uint2*>(tp);
        const uint2 a1 = *reinterpret_cast<const uint2*>(tp + 16);
        const v8bf av = __builtin_bit_cast(v8bf, make_uint4(a0.x, a0.y, a1.x, a1.y));
        o[8 * bb + nt] = mfma_bf16(av, pbh, o[8 * bb + nt]);
        o[8 * bb + nt] = mfma_bf16(av, pbl, o[8 * bb + nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // step k: wait for its copies, barrier (they are visible, and step k - 1's
  // compute is done with ct, tr and stage (k - 1) % NS), copy step k + NS - 1
  // into that stage, convert, barrier, compute
  const int nsteps = lo < hi ? (hi - lo + PT - 1) / PT : 0;
  for (int j = 0; j < NS - 1 && j < nsteps; ++j) issue(j, lo + j * PT);
  for (int k = 0; k < nsteps; ++k) {
    const int st = k % NS, p0 = lo + k * PT;
    vm_wait(n_copies * min(NS - 2, nsteps - 1 - k));
    __syncthreads();
    if (k + NS - 1 < nsteps) issue((k + NS - 1) % NS, p0 + (NS - 1) * PT);
    convert(st);
    __syncthreads();
    // scores (waves whose token sees this step), exchange, values (pairs
    // with a member that sees it; an idle member contributes p = 0)
    float ps[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float alpha = 1.f;
    if (active && p0 < my_end) scores(st, p0, ps, alpha);
#pragma unroll
    for (int j = 0; j < 8; ++j) xbuf[wave][j][lane] = ps[j >> 2][j & 3];
    xbuf[wave][8][lane] = alpha;
    __syncthreads();
    if (p0 < pair_end) values(st);
  }
  if (pair_end == 0) return;
  // lane l writes O^T of pair column l mod 16 (when its member is active),
  // latent features 256 pm + 16 nt + 4 q4 + i
  const int cw = (wave & ~1) | (l16 >> 3);
  if (kv_sh[cw] > 0) {
    const size_t cidx = ((size_t)split * g.T + tok_sh[cw]) * g.H + head_sh[cw] + (l16 & 7);
    float* po = g.part_o + cidx * DL + 256 * pm;
#pragma unroll
    for (int nt = 0; nt < DL / 32; ++nt)
      *reinterpret_cast<float4*>(po + 16 * nt + 4 * q4) =
          make_float4(o[nt][0], o[nt][1], o[nt][2], o[nt][3]);
  }
  float ltot = lrun + __shfl_xor(lrun, 16);
  ltot += __shfl_xor(ltot, 32);
  if (active && !lo_col && q4 == 0) {
    const size_t pidx = ((size_t)split * g.T + t) * g.H + h;
    g.part_ml[pidx * 2] = mrun;
    g.part_ml[pidx * 2 + 1] = ltot;
  }
}

// ------------------------------------ query absorption, value up-projection
// Both are dense bf16 MFMA products per head.  The weight codes are exact in
// bf16 (pre-converted by mla_pack_ukv_kernel); an fp32 activation a is split
// into its bf16 high part and the bf16 rounding of a - high, and both halves
// go through the MFMA into one fp32 accumulator (the product of the two is
// within about 2^-17 of the fp32 one, sums in fp32).

// e4m3 codes of the key-value up-projection (per head: 128 key rows, 128
// value rows, 512 latents) -> bf16 copies: ukt[h][r][d] = W_uk[d][r] (the
// key rows transposed, so a latent's 128 weights are contiguous),
// uv[h][d][r] = W_uv[d][r] and uk[h][d][r] = W_uk[d][r].
__global__ __launch_bounds__(256) void mla_pack_ukv_kernel(int H, const uint8_t* __restrict__ w_kvb,
                                                           uint16_t* __restrict__ ukt,
                                                           uint16_t* __restrict__ uv,
                                                           uint16_t* __restrict__ uk) {
  const size_t n = (size_t)H * DN * DL;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < 3 * n;
       i += (size_t)gridDim.x * 256) {
    const int part = (int)(i / n);
    const size_t j = i - part * n;
    const int h = (int)(j / (DN * DL)), rem = (int)(j % (DN * DL));
    if (part == 0) {
      const int r = rem / DN, d = rem % DN;   // output [h][r][d]
      const float v = e4m3_val(w_kvb[((size_t)h * (DN + DV) + d) * DL + r]);
      ukt[j] = (uint16_t)(__float_as_uint(v) >> 16);
    } else {
      const int d = rem / DL, r = rem % DL;   // output [h][d][r]
      const float v = e4m3_val(w_kvb[((size_t)h * (DN + DV) + (part == 1 ? DN : 0) + d) * DL + r]);
      (part == 1 ? uv : uk)[j] = (uint16_t)(__float_as_uint(v) >> 16);
    }
  }
}


// q: the q_b projection as nsplit K-slice partial sums [nsplit, T, H*192],
// added in slice order (the order of launch_slice_sum).
// qcat[t, h] = scale * [W_uk^T q_nope (512), rope(q_pe) (64)] in fp32, per
// latent block b: s_b * sum_d code[d][r] q[d] (W_uk of head h: key-value
// up-projection rows h*(DN+DV) .. + DN - 1, one 128-row scale block).
// Workgroup = (head, TB tokens); wave w: latents 128 w .. + 127 (block w).
// TB = 16 for small batches (decode), so that 64 heads give 256 workgroups
// at 64 tokens; 32 otherwise (each head's W_uk fragments feed twice the MFMAs).
template <int TB>
__global__ __launch_bounds__(256) void mla_qabsorb_kernel(
    int T, int H, int nsplit, float smscale, const float* __restrict__ q,
    const uint16_t* __restrict__ ukt,
    const float* __restrict__ s_kvb, const double* __restrict__ inv_freq,
    const int32_t* __restrict__ cached_len, int n_new, int max_len,
    float* __restrict__ qcat) {
  constexpr int MT = TB / 16;
  const int h = blockIdx.x, t0 = blockIdx.y * TB, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, q4 = lane >> 4, l16 = lane & 15;
  const int qld = H * (DN + DR);
  const size_t slice = (size_t)T * qld;
  auto q4sum = [&](const float* p) {   // the partial sums of 4 values, in slice order
    float4 a = *reinterpret_cast<const float4*>(p);
    for (int s = 1; s < nsplit; ++s) {
      const float4 b = *reinterpret_cast<const float4*>(p + s * slice);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    return a;
  };
  // A: q_nope of tokens t0 + 16 mt + l16 (the last token repeated past T),
  // features 32 ks + 8 q4 .. + 7
  v8bf ahi[MT][DN / 32], alo[MT][DN / 32];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = min(t0 + 16 * mt + l16, T - 1);
    const float* qp = q + (size_t)t * qld + h * (DN + DR) + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < DN / 32; ++ks)
      split8(q4sum(qp + 32 * ks), q4sum(qp + 32 * ks + 4), &ahi[mt][ks], &alo[mt][ks]);
  }
  v4f acc[MT][8] = {};
  const uint16_t* bp = ukt + ((size_t)h * DL + 128 * wave + l16) * DN + 8 * q4;
#pragma unroll
  for (int ks = 0; ks < DN / 32; ++ks) {
    v8bf b[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      b[ct] = __builtin_bit_cast(v8bf,
                                 *reinterpret_cast<const uint4*>(bp + (size_t)16 * ct * DN + 32 * ks));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][ct] = mfma_bf16(ahi[mt][ks], b[ct], acc[mt][ct]);
        acc[mt][ct] = mfma_bf16(alo[mt][ks], b[ct], acc[mt][ct]);
      }
  }
  // lane: latent 128 w + 16 ct + l16, tokens 16 mt + 4 q4 + i
  const float sk = s_kvb[(size_t)(2 * h) * (DL / QBLK) + wave];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * mt + 4 * q4 + i;
      if (t >= T) continue;
      float* dst = qcat + ((size_t)t * H + h) * DQ + 128 * wave + l16;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) dst[16 * ct] = acc[mt][ct][i] * sk * smscale;
    }
  // rotary part: thread (token tt, pair i)
  for (int i = tid; i < TB * (DR / 2); i += 256) {
    const int tt = i / (DR / 2), pr = i % (DR / 2), t = t0 + tt;
    if (t >= T) continue;
    int seq;
    const int pos = token_pos(cached_len, t, n_new, max_len, &seq);
    const float* qp = q + (size_t)t * qld + h * (DN + DR) + DN;
    float qa = qp[2 * pr], qb = qp[2 * pr + 1];
    for (int s = 1; s < nsplit; ++s) {
      qa += qp[s * slice + 2 * pr];
      qb += qp[s * slice + 2 * pr + 1];
    }
    float ra, rb;
    rope_pair(qa, qb, pos, inv_freq[pr], &ra, &rb);
    float* dst = qcat + ((size_t)t * H + h) * DQ + DL;
    dst[2 * pr] = ra * smscale;
    dst[2 * pr + 1] = rb * smscale;
  }
}

constexpr int VA_LD = DL + 8;         // bf16 stride of an activation row in LDS

// For head h and TB tokens (16 or 32): merge the position splits (m, l, O) into
// o_lat = sum_j p_j c_j / sum_j p_j, apply W_uv (rows h*(DN+DV)+DN .. + DV - 1,
// one 128-row scale block) as sum_r code[d][r] (s_(r/128) o_lat[r]), write the
// 128 outputs as one 1x128 block of the output projection's input (codes +
// scale) and, if attn != null, as fp32.  Wave w: outputs 32 w .. + 31.
template <int TB>
__global__ __launch_bounds__(256) void mla_vup_kernel(
    int T, int H, int nsplit, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const uint16_t* __restrict__ uv, const float* __restrict__ s_kvb,
    uint8_t* __restrict__ o_q, float* __restrict__ o_s, float* __restrict__ attn) {
  constexpr int MT = TB / 16;
  const int h = blockIdx.x, t0 = blockIdx.y * TB, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, q4 = lane >> 4, l16 = lane & 15;
  __shared__ __attribute__((aligned(16))) uint16_t a_hi[TB * VA_LD];
  __shared__ __attribute__((aligned(16))) uint16_t a_lo[TB * VA_LD];
  __shared__ float bmax[4][TB];
  const float* sv = s_kvb + (size_t)(2 * h + 1) * (DL / QBLK);
  // merge: thread = (token tt, 16 consecutive latents)
  for (int it = tid; it < TB * (DL / 16); it += 256) {
    const int tt = it / (DL / 16), r0 = 16 * (it % (DL / 16)), t = t0 + tt;
    float a[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) a[j] = 0.f;
    if (t < T) {
      float M = -INFINITY;
      for (int s = 0; s < nsplit; ++s)
        M = fmaxf(M, part_ml[(((size_t)s * T + t) * H + h) * 2]);
      float L = 0.f;
      for (int s = 0; s < nsplit; ++s) {
        const size_t pi = ((size_t)s * T + t) * H + h;
        const float m = part_ml[pi * 2];
        if (m == -INFINITY) continue;
        const float wgt = __expf(m - M);
        L += part_ml[pi * 2 + 1] * wgt;
        const float4* po = reinterpret_cast<const float4*>(part_o + pi * DL + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v = po[j];
          a[4 * j] += v.x * wgt;
          a[4 * j + 1] += v.y * wgt;
          a[4 * j + 2] += v.z * wgt;
          a[4 * j + 3] += v.w * wgt;
        }
      }
      const float sc = sv[r0 / QBLK];
#pragma unroll
      for (int j = 0; j < 16; ++j) a[j] = (a[j] / L) * sc;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      v8bf hi, lo;
      split8(make_float4(a[8 * half], a[8 * half + 1], a[8 * half + 2], a[8 * half + 3]),
             make_float4(a[8 * half + 4], a[8 * half + 5], a[8 * half + 6], a[8 * half + 7]),
             &hi, &lo);
      *reinterpret_cast<v8bf*>(&a_hi[tt * VA_LD + r0 + 8 * half]) = hi;
      *reinterpret_cast<v8bf*>(&a_lo[tt * VA_LD + r0 + 8 * half]) = lo;
    }
  }
  __syncthreads();
  // out[t, d]: A = activation halves (tokens 16 mt + l16, latents 32 ks + 8 q4
  // ..), B = W_uv rows d = 32 w + 16 ct + l16
  v4f acc[MT][2] = {};
  const uint16_t* bp = uv + ((size_t)h * DV + 32 * wave + l16) * DL + 8 * q4;
#pragma unroll 4
  for (int ks = 0; ks < DL / 32; ++ks) {
    v8bf b[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
      b[ct] = __builtin_bit_cast(v8bf,
                                 *reinterpret_cast<const uint4*>(bp + (size_t)16 * ct * DL + 32 * ks));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int ao = (16 * mt + l16) * VA_LD + 32 * ks + 8 * q4;
      const v8bf ah = *reinterpret_cast<const v8bf*>(&a_hi[ao]);
      const v8bf al = *reinterpret_cast<const v8bf*>(&a_lo[ao]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[mt][ct] = mfma_bf16(ah, b[ct], acc[mt][ct]);
        acc[mt][ct] = mfma_bf16(al, b[ct], acc[mt][ct]);
      }
    }
  }
  // lane: outputs d = 32 w + 16 ct + l16 of tokens 16 mt + 4 q4 + i; block
  // maxima over the 128 outputs of a token (16 lanes x 2 tiles x 4 waves)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = fmaxf(fabsf(acc[mt][0][i]), fabsf(acc[mt][1][i]));
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) m = fmaxf(m, __shfl_xor(m, x));
      if (l16 == 0) bmax[wave][16 * mt + 4 * q4 + i] = m;
    }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = 16 * mt + 4 * q4 + i, t = t0 + tt;
      if (t >= T) continue;
      const float amax = fmaxf(fmaxf(bmax[0][tt], bmax[1][tt]), fmaxf(bmax[2][tt], bmax[3][tt]));
      const float s = fp8_scale(amax);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int d = 32 * wave + 16 * ct + l16;
        const float v = acc[mt][ct][i];
        const uint32_t c = cvt4_e4m3(clamp_fp8(v / s), 0.f, 0.f, 0.f);
        o_q[(size_t)t * H * DV + h * DV + d] = (uint8_t)(c & 0xFFu);
        if (attn) attn[(size_t)t * H * DV + h * DV + d] = v;
      }
      if (wave == 0 && l16 == 0) o_s[(size_t)t * H + h] = s;
    }
}

}  // namespace

// ------------------------------------------------------------- launchers
hipError_t launch_pack_rows(int n_pad, int K, const uint8_t* src0, int n0, const uint8_t* src1,
                            int n1, const float* s0, const float* s1, uint8_t* dst_codes,
                            float* dst_scales, hipStream_t s) {
  const long n = (long)n_pad * K / 16;
  pack_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n_pad, K, src0, n0, src1, n1,
                                                               dst_codes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int kb = K / QBLK, nb = n_pad / QBLK;
  pack_row_scales_kernel<<<(nb * kb + 255) / 256, 256, 0, s>>>(
      nb, kb, s0, (n0 + QBLK - 1) / QBLK, s1, (n1 + QBLK - 1) / QBLK, dst_scales);
  return hipGetLastError();
}

hipError_t launch_dense_tiles(int T, int bm, int32_t* offsets, int32_t* mt_start,
                              int32_t* tile_group, hipStream_t s) {
  const int n = (T + bm - 1) / bm;
  dense_tiles_kernel<<<(max(n, 1) + 255) / 256, 256, 0, s>>>(T, bm, offsets, mt_start,
                                                              tile_group);
  return hipGetLastError();
}

hipError_t launch_slice_sum(int T, int ncol, int ld, int nsplit, const float* part,
                            const uint16_t* residual, void* out, int out_ld, hipStream_t s) {
  const long n = (long)T * (ncol / 4);
  slice_sum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(T, ncol, ld, nsplit, part,
                                                               residual, out, out_ld);
  return hipGetLastError();
}

hipError_t launch_mla_latent(int T, int nsplit, int q_lora, int qkv_ld, float eps,
                             const float* qkv, const uint16_t* g_qa, const uint16_t* g_kva,
                             const double* inv_freq, const int32_t* cached_len, int n_new,
                             int max_len, uint8_t* qa_q, float* qa_s, uint8_t* c_codes,
                             float* c_scales, uint16_t* c_rope, double* rot, hipStream_t s) {
  if (q_lora + DL + DR > MAX_QKV) return hipErrorInvalidValue;
  mla_latent_kernel<<<T, 256, 0, s>>>(T, nsplit, q_lora, qkv_ld, eps, qkv, g_qa, g_kva, inv_freq,
                                      cached_len, n_new, max_len, qa_q, qa_s, c_codes, c_scales,
                                      c_rope, rot);
  return hipGetLastError();
}

hipError_t launch_mla_pack_ukv(int H, const uint8_t* w_kvb, uint16_t* ukt, uint16_t* uv,
                              uint16_t* uk, hipStream_t s) {
  mla_pack_ukv_kernel<<<1024, 256, 0, s>>>(H, w_kvb, ukt, uv, uk);
  return hipGetLastError();
}

hipError_t launch_mla_qabsorb(int T, int H, int nsplit, float smscale, const float* q,
                              const uint16_t* ukt, const float* s_kvb, const double* inv_freq,
                              const int32_t* cached_len, int n_new, int max_len, float* qcat,
                              hipStream_t s) {
  // 16-token tiles while 32-token ones would leave CUs idle
  if ((long)H * ((T + 31) / 32) < 256) {
    dim3 grid(H, (T + 15) / 16);
    mla_qabsorb_kernel<16><<<grid, 256, 0, s>>>(T, H, nsplit, smscale, q, ukt, s_kvb, inv_freq,
                                                cached_len, n_new, max_len, qcat);
  } else {
    dim3 grid(H, (T + 31) / 32);
    mla_qabsorb_kernel<32><<<grid, 256, 0, s>>>(T, H, nsplit, smscale, q, ukt, s_kvb, inv_freq,
                                                cached_len, n_new, max_len, qcat);
  }
  return hipGetLastError();
}

hipError_t launch_mla_attn(int T, int H, int n_seq, int n_new, int max_len, int nsplit,
                           int chunk, const uint8_t* c_codes, const float* c_scales,
                           const uint16_t* c_rope, const float* qcat,
                           const int32_t* cached_len, float* part_o, float* part_ml,
                           hipStream_t s) {
  AttnArgs a{};
  a.c_codes = c_codes;
  a.c_scales = c_scales;
  a.c_rope = c_rope;
  a.qcat = qcat;
  a.cached_len = cached_len;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.T = T;
  a.H = H;
  a.n_new = n_new;
  a.max_len = max_len;
  a.nsplit = nsplit;
  a.chunk = chunk;
  a.items_per_split = mla_attn_items(T, H, n_seq, n_new, &a.mode, &a.hw);
  mla_attn_kernel<<<a.items_per_split * nsplit, 512, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_mla_vup(int T, int H, int nsplit, const float* part_o, const float* part_ml,
                          const uint16_t* uv, const float* s_kvb, uint8_t* o_q, float* o_s,
                          float* attn, hipStream_t s) {
  if ((long)H * ((T + 31) / 32) < 256) {
    dim3 grid(H, (T + 15) / 16);
    mla_vup_kernel<16><<<grid, 256, 0, s>>>(T, H, nsplit, part_o, part_ml, uv, s_kvb, o_q, o_s,
                                            attn);
  } else {
    dim3 grid(H, (T + 31) / 32);
    mla_vup_kernel<32><<<grid, 256, 0, s>>>(T, H, nsplit, part_o, part_ml, uv, s_kvb, o_q, o_s,
                                            attn);
  }
  return hipGetLastError();
}

}  // namespace k2
