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

// ------------------------------------------------------- latent attention
// A workgroup covers 64 columns, each a (token, head) pair: mode 0 (one new
// token per sequence) one token's heads, mode 1 up to 8 consecutive new
// tokens of one sequence x 8 heads.  The cache positions [lo, hi) of its
// split are visited in steps of 32, by two kinds of waves that work one step
// apart:
//  - score waves 0-3, 16 columns each: S^T = C Q^T over a step's 576 cached
//    features, then the online softmax of their columns; the probabilities
//    and rescale factors go to LDS.  The cache codes are read as e4m3 bytes
//    and converted to exact bf16 in registers, and every cache fragment feeds
//    the MFMAs of both 8-column halves of the wave.
//  - value waves 4-7, latent block b = wave - 4 (128 features): convert block
//    b of the previous step's codes into a private transposed bf16 tile, then
//    O^T[latent, column] += C_b^T (p scale_b)^T for all 64 columns, so every
//    cache fragment feeds 8 MFMAs.
// A SIMD holds one wave of each kind, in different phases.  The cache bytes
// of a step (codes, rotary keys, scales) are copied straight into one of four
// LDS stages by global_load_lds, two steps ahead; one barrier per step
// orders the copies, the probabilities of the step before and the reuse of
// a stage.
//
// Sums to fp32 precision: a score wave's 16 MFMA columns per half are 8
// columns x {hi, lo}, the bf16 high part of a query and the bf16 rounding of
// its remainder, so one MFMA gives both halves of the product and the two
// columns add to it within about 2^-17 relative.  Per 128-latent block b:
//   S_b^T = C_b Q^T; s = sum_b scale_b(pos) S_b + S_rope
//   O_b^T += C_b^T (p scale_b)^T as two MFMAs per fragment, the high and the
//            low bf16 halves of p scale_b
// and finally O^T (column x 512), the reference maximum m and the sum l are
// written unscaled for the split merge.
struct AttnArgs {
  const uint8_t* c_codes;
  const float* c_scales;
  const uint16_t* c_rope;
  const uint16_t* qcat;      // [T, H, 2, 576]: bf16 high parts, then the bf16 roundings of
                             // the remainders, of the queries with the softmax scale folded in
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

constexpr int AW = 8;        // waves per workgroup
constexpr int SW = 4;        // score waves (the others are value waves, one per latent block)
constexpr int ACOLS = 64;    // columns per workgroup
constexpr int NSR = 4;       // LDS stages of raw cache bytes (copies run two steps ahead)
constexpr float LAZY_E = 5.5451774f;   // 8 ln 2: margin before a column's reference maximum moves
// one stage: codes of 16 position pairs, each pair's two 512-byte rows
// followed by 16 bytes of padding; rotary keys [32][64] bf16 (chunks
// swizzled); scales [4][32]
constexpr int CPAIR = 2 * DL + 16;
constexpr int SG_ROPE = (PT / 2) * CPAIR, SG_SC = SG_ROPE + PT * DR * 2,
              SG = SG_SC + (DL / QBLK) * PT * 4;
// probabilities of a column: 32 positions, row stride 36 floats (the 16
// columns a value wave reads at once fall on distinct banks)
constexpr int PB_LD = PT + 4;
// a value wave's transposed bf16 tile: latent rows of 32 positions at a
// stride of 40 (80 bytes: the 16 rows of a fragment read on distinct banks),
// 16-row blocks 16 dwords apart in bank (the four blocks a conversion
// instruction writes do not collide)
constexpr int TW_LD = PT + 8, TW_BLK = 16 * TW_LD + 32, TW_ELEMS = 8 * TW_BLK;

// byte offset in a stage of the 16-byte code chunk c of position p: the pair
// padding puts consecutive pairs 4 banks apart, and an odd position's chunks
// are swapped in halves of 8 (slot c ^ 8), so 16 consecutive positions (a
// score fragment) and the 16 even or odd positions of a conversion
// instruction read distinct banks.  The swap only adds or subtracts 128
// bytes, so a fragment's address is a per-lane base plus a constant.
__device__ __forceinline__ int code_off(int c, int p) {
  return (p >> 1) * CPAIR + (p & 1) * DL + 16 * (c ^ ((p & 1) << 3));
}

// 8 e4m3 codes (two dwords) -> 8 exact bf16 values
__device__ __forceinline__ v8bf codes_bf16(uint2 w) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true));
  return __builtin_bit_cast(v8bf, make_uint4(a, b, c, d));
}

__global__ __launch_bounds__(512, 1) void mla_attn_kernel(const AttnArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[NSR][SG];
  __shared__ __attribute__((aligned(16))) uint16_t tw_all[AW - SW][TW_ELEMS];
  __shared__ __attribute__((aligned(16))) float pbuf[2][ACOLS * PB_LD];
  __shared__ float abuf[2][ACOLS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, l16 = lane & 15;
  const int item = blockIdx.x % g.items_per_split, split = blockIdx.x / g.items_per_split;

  // column c -> (token, head); false for columns past the heads or tokens
  int tok0 = 0, h0 = 0, seq = 0;
  if (g.mode == 0) {
    const int ngrp = g.H / g.hw;
    tok0 = item / ngrp;
    h0 = (item % ngrp) * g.hw;
  } else {
    const int hg_n = g.H / 8;
    const int per_seq = ((g.n_new + 7) / 8) * hg_n;
    const int s_ = item / per_seq, rem = item % per_seq;
    tok0 = s_ * g.n_new + (rem / hg_n) * 8;   // first token of the block
    h0 = (rem % hg_n) * 8;
  }
  auto column = [&](int c, int* t, int* h) -> bool {
    if (g.mode == 0) {
      *t = tok0;
      *h = min(h0 + c, g.H - 1);
      return c < g.hw;
    }
    const int ti = (tok0 % g.n_new) + c / 8;
    *t = tok0 + min(c / 8, g.n_new - 1 - tok0 % g.n_new);
    *h = h0 + (c & 7);
    return ti < g.n_new;
  };
  // the workgroup's positions: its split's range, up to the last visible one
  // of its last token
  int t_last, h_unused;
  column(g.mode == 0 ? 0 : ACOLS - 1, &t_last, &h_unused);
  const int wg_end = token_pos(g.cached_len, t_last, g.n_new, g.max_len, &seq) + 1;
  const int lo = split * g.chunk, hi = min(wg_end, lo + g.chunk);
  const int nsteps = lo < hi ? (hi - lo + PT - 1) / PT : 0;
  const size_t cbase = (size_t)seq * g.max_len;
  const uint8_t* codes_seq = g.c_codes + cbase * DL;
  const uint16_t* rope_seq = g.c_rope + cbase * DR;
  const float* sc_seq = g.c_scales + cbase * (DL / QBLK);

  // copies of the step at p0 into stage st; positions past hi copy position
  // hi - 1 (written, finite), which the mask and p = 0 leave without effect.
  // Wave w: code instructions 2w, 2w + 1 (two positions each), waves 0-3 one
  // rotary instruction (8 positions), waves 4-5 one scale instruction (two
  // blocks): 3 copies per step for waves 0-5, 2 for waves 6-7
  const int n_copies = wave < 6 ? 3 : 2;
  auto issue = [&](int st, int p0) {
    const int plast = hi - 1;
    uint8_t* sb = stg[st];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * wave + u;
      const int p = 2 * i + (lane >> 5);
      const int pc = min(p0 + p, plast);
      const int c = (lane & 31) ^ ((lane >> 5) << 3);   // the chunk that lands in slot lane % 32
      lds_copy16(codes_seq, (uint32_t)(pc * DL + 16 * c), lds_addr(sb + i * CPAIR));
    }
    if (wave < 4) {
      const int p = 8 * wave + (lane >> 3);
      const int pc = min(p0 + p, plast);
      const int c = (lane & 7) ^ ((p >> 1) & 7);
      lds_copy16(rope_seq, (uint32_t)(pc * DR * 2 + 16 * c), lds_addr(sb + SG_ROPE + wave * 1024));
    } else if (wave < 6) {
      const int i = wave - 4, blk = 2 * i + (lane >> 5);
      const int pc = min(p0 + (lane & 31), plast);
      lds_copy4(sc_seq, (uint32_t)((pc * (DL / QBLK) + blk) * 4),
                lds_addr(sb + SG_SC + 2 * i * PT * 4));
    }
  };

  // probabilities start at 0 and rescale factors at 1 (columns no score wave
  // owns keep them)
  for (int i = tid; i < 2 * ACOLS * PB_LD; i += AW * 64) (&pbuf[0][0])[i] = 0.f;
  if (tid < 2 * ACOLS) (&abuf[0][0])[tid] = 1.f;
  if (nsteps > 0) issue(0, lo);
  if (nsteps > 1) issue(1, lo + PT);

  if (wave < SW) {
    // ------------------------------------------------------ score wave
    // column of this lane in half ct: 16 wave + 8 ct + l16 % 8, high query
    // halves in lanes l16 < 8, low halves in l16 >= 8 (a column past the
    // heads or tokens reads a valid query and is masked)
    int ctok[2], chead[2], cend[2];
    bool cact[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      cact[ct] = column(16 * wave + 8 * ct + (l16 & 7), &ctok[ct], &chead[ct]);
      int sq;
      cend[ct] = cact[ct] ? token_pos(g.cached_len, ctok[ct], g.n_new, g.max_len, &sq) + 1 : 0;
    }
    const bool wave_on = __builtin_amdgcn_readfirstlane(
                             (int)(__builtin_amdgcn_ballot_w64(cact[0] || cact[1]) != 0)) != 0;
    // the queries as B fragments (dims 32 ks + 8 q4 .. + 7)
    v8bf qb[2][DQ / 32];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint16_t* qp = g.qcat + ((size_t)ctok[ct] * g.H + chead[ct]) * (2 * DQ) +
                           (l16 >= 8 ? DQ : 0) + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks)
        qb[ct][ks] = *reinterpret_cast<const v8bf*>(qp + 32 * ks);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

    for (int j = 0; j <= nsteps; ++j) {
      if (j < nsteps) vm_wait(j + 1 < nsteps ? n_copies : 0);
      __syncthreads();
      if (j + 2 < nsteps) issue((j + 2) % NSR, lo + (j + 2) * PT);
      if (j == nsteps || !wave_on) continue;
      const uint8_t* sb = stg[j % NSR];
      const float* scb = reinterpret_cast<const float*>(sb + SG_SC);
      const int p0 = lo + j * PT;
      // S^T[pos, column] for positions p0 + 16 pt + 4 q4 + i, in ten fragment
      // groups per step: for each 16-position tile pt, the four latent blocks
      // (four e4m3 fragments each) and the rotary key (two bf16 fragments);
      // group u + 1's fragments are read while group u's MFMAs run
      // (a group's fragments: four e4m3 ones, 2 dwords each, or two bf16
      // rotary ones, 4 dwords each)
      auto kload = [&](int u, uint2 (&w)[4]) {
        const int pt = u / 5, k = u % 5, p = 16 * pt + l16;
        if (k < DL / QBLK) {
          // chunk c = 8 k + 2 kk + q4 / 2: bit 3 of c is k % 2, so its slot
          // c ^ 8 (p % 2) is c + 8 (p % 2) for even k, c - 8 (p % 2) for odd k
          const int odd = (p & 1) * 128;
          const uint8_t* rowp = sb + (p >> 1) * CPAIR + (p & 1) * DL + 8 * (q4 & 1) +
                                16 * (q4 >> 1) + ((k & 1) ? -odd : odd);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            w[kk] = *reinterpret_cast<const uint2*>(rowp + 16 * (8 * k + 2 * kk));
        } else {
#pragma unroll
          for (int kr = 0; kr < DR / 32; ++kr) {
            const uint4 r = *reinterpret_cast<const uint4*>(
                sb + SG_ROPE + p * DR * 2 + 16 * ((4 * kr + q4) ^ ((p >> 1) & 7)));
            w[2 * kr] = make_uint2(r.x, r.y);
            w[2 * kr + 1] = make_uint2(r.z, r.w);
          }
        }
      };
      v4f s[2][2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) s[pt][0] = s[pt][1] = v4f{0.f, 0.f, 0.f, 0.f};
      uint2 wc[4], wn[4];
      kload(0, wc);
#pragma unroll
      for (int u = 0; u < 10; ++u) {
        if (u + 1 < 10) kload(u + 1, wn);
        __builtin_amdgcn_sched_barrier(0);
        const int pt = u / 5, k = u % 5;
        if (k < DL / QBLK) {
          v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const v8bf a = codes_bf16(wc[kk]);
            a0 = mfma_bf16(a, qb[0][4 * k + kk], a0);
            a1 = mfma_bf16(a, qb[1][4 * k + kk], a1);
          }
          const float4 sc = *reinterpret_cast<const float4*>(scb + k * PT + 16 * pt + 4 * q4);
          s[pt][0][0] = fmaf(sc.x, a0[0], s[pt][0][0]);
          s[pt][0][1] = fmaf(sc.y, a0[1], s[pt][0][1]);
          s[pt][0][2] = fmaf(sc.z, a0[2], s[pt][0][2]);
          s[pt][0][3] = fmaf(sc.w, a0[3], s[pt][0][3]);
          s[pt][1][0] = fmaf(sc.x, a1[0], s[pt][1][0]);
          s[pt][1][1] = fmaf(sc.y, a1[1], s[pt][1][1]);
          s[pt][1][2] = fmaf(sc.z, a1[2], s[pt][1][2]);
          s[pt][1][3] = fmaf(sc.w, a1[3], s[pt][1][3]);
        } else {
#pragma unroll
          for (int kr = 0; kr < DR / 32; ++kr) {
            const v8bf a = __builtin_bit_cast(
                v8bf, make_uint4(wc[2 * kr].x, wc[2 * kr].y, wc[2 * kr + 1].x, wc[2 * kr + 1].y));
            s[pt][0] = mfma_bf16(a, qb[0][DL / 32 + kr], s[pt][0]);
            s[pt][1] = mfma_bf16(a, qb[1][DL / 32 + kr], s[pt][1]);
          }
        }
        if (u + 1 < 10) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) wc[kk] = wn[kk];
        }
      }
      // per half: the two columns of a pair add to its score; mask; lazy
      // reference maximum; probabilities
      float* pb = pbuf[j & 1];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float v[8];
        float mx = -INFINITY;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = p0 + 16 * pt + 4 * q4 + i;
            float x = s[pt][ct][i] + xor8(s[pt][ct][i]);
            if (pos >= cend[ct] || pos >= hi) x = -INFINITY;
            v[4 * pt + i] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // the reference maximum moves only when the step's maximum passes it
        // by more than LAZY_E, so the probabilities stay below e^LAZY_E and
        // the outputs are rarely rescaled; the merge and the normalisation use
        // the same reference, which cancels.  A column that has seen no
        // position yet keeps p = 0.
        const float mnew = mx > mrun[ct] + LAZY_E ? mx : mrun[ct];
        const bool none = mnew == -INFINITY;
        const float alpha = none ? 1.f : __expf(mrun[ct] - mnew);
        float lsum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[k] = none ? 0.f : __expf(v[k] - mnew);
          lsum += v[k];
        }
        lrun[ct] = lrun[ct] * alpha + lsum;
        mrun[ct] = mnew;
        if (l16 < 8) {
          const int c = 16 * wave + 8 * ct + l16;
#pragma unroll
          for (int pt = 0; pt < 2; ++pt)
            *reinterpret_cast<float4*>(&pb[c * PB_LD + 16 * pt + 4 * q4]) =
                make_float4(v[4 * pt], v[4 * pt + 1], v[4 * pt + 2], v[4 * pt + 3]);
          if (q4 == 0) abuf[j & 1][c] = alpha;
        }
      }
    }
    // m and l of each column (the four lanes of a column add their sums)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float ltot = lrun[ct] + __shfl_xor(lrun[ct], 16);
      ltot += __shfl_xor(ltot, 32);
      if (cact[ct] && l16 < 8 && q4 == 0) {
        const size_t pidx = ((size_t)split * g.T + ctok[ct]) * g.H + chead[ct];
        g.part_ml[pidx * 2] = mrun[ct];
        g.part_ml[pidx * 2 + 1] = ltot;
      }
    }
  } else {
    // ------------------------------------------------------ value wave
    const int b = wave - SW;   // latent block
    uint16_t* tw = tw_all[b];
    v4f o[8][4];   // O^T: latent 128 b + 16 r + 4 q4 + i, column 16 c4 + l16
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) o[r][c4] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j <= nsteps; ++j) {
      if (j < nsteps) vm_wait(j + 1 < nsteps ? n_copies : 0);
      __syncthreads();
      if (j + 2 < nsteps) issue((j + 2) % NSR, lo + (j + 2) * PT);
      if (j == 0) continue;
      // step j - 1
      const uint8_t* sb = stg[(j - 1) % NSR];
      const float* scb = reinterpret_cast<const float*>(sb + SG_SC);
      // block b's codes -> tw: lane = (position pair l16, chunk (lane / 16) +
      // 4 k of the block); row 16 cl + e holds latent 128 b + 16 cl + e at
      // positions 0..31
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cl = q4 + 4 * k, c = 8 * b + cl;
        uint32_t pk[2][8];   // bf16 pairs: codes 2e, 2e + 1 of position 2 l16 + jj
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int p = 2 * l16 + jj;
          const uint4 cv = *reinterpret_cast<const uint4*>(sb + code_off(c, p));
          const uint32_t w4[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pk[jj][2 * e] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[e], 1.f, false));
            pk[jj][2 * e + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[e], 1.f, true));
          }
        }
        uint16_t* dst = tw + cl * TW_BLK + 2 * l16;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int w = e >> 1;
          const uint32_t v = (e & 1) ? ((pk[0][w] >> 16) | (pk[1][w] & 0xFFFF0000u))
                                     : ((pk[0][w] & 0xFFFFu) | (pk[1][w] << 16));
          *reinterpret_cast<uint32_t*>(dst + e * TW_LD) = v;
        }
      }
      // (the tile is this wave's: its own writes above precede its reads)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // B: p scale_b at positions 8 q4 .. + 7 of column 16 c4 + l16, as high
      // and low bf16 halves
      const float* pb = pbuf[(j - 1) & 1];
      const float4 s0 = *reinterpret_cast<const float4*>(scb + b * PT + 8 * q4);
      const float4 s1 = *reinterpret_cast<const float4*>(scb + b * PT + 8 * q4 + 4);
      v8bf ph[4], pl[4];
      float al[4];
      bool moved = false;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const float* pr = pb + (16 * c4 + l16) * PB_LD + 8 * q4;
        const float4 x0 = *reinterpret_cast<const float4*>(pr);
        const float4 x1 = *reinterpret_cast<const float4*>(pr + 4);
        split8(make_float4(x0.x * s0.x, x0.y * s0.y, x0.z * s0.z, x0.w * s0.w),
               make_float4(x1.x * s1.x, x1.y * s1.y, x1.z * s1.z, x1.w * s1.w), &ph[c4], &pl[c4]);
        al[c4] = abuf[(j - 1) & 1][16 * c4 + l16];
        moved = moved || al[c4] != 1.f;
      }
      // rescale only when some column's reference moved (alpha = 1 leaves them)
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) o[r][c4] *= al[c4];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const v8bf a = *reinterpret_cast<const v8bf*>(tw + r * TW_BLK + l16 * TW_LD + 8 * q4);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) o[r][c4] = mfma_bf16(a, ph[c4], o[r][c4]);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) o[r][c4] = mfma_bf16(a, pl[c4], o[r][c4]);
      }
    }
    // O^T of the columns this workgroup owns
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      int t, h;
      if (!column(16 * c4 + l16, &t, &h)) continue;
      float* po = g.part_o + (((size_t)split * g.T + t) * g.H + h) * DL + QBLK * b + 4 * q4;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        *reinterpret_cast<float4*>(po + 16 * r) =
            make_float4(o[r][c4][0], o[r][c4][1], o[r][c4][2], o[r][c4][3]);
    }
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
    uint16_t* __restrict__ qcat) {
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
      uint16_t* dst = qcat + ((size_t)t * H + h) * (2 * DQ) + 128 * wave + l16;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const float v = acc[mt][ct][i] * sk * smscale;
        dst[16 * ct] = (uint16_t)bf16_half2(v, 0.f, 0.f);
        dst[DQ + 16 * ct] = (uint16_t)bf16_half2(v, 0.f, 1.f);
      }
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
    uint32_t* dst = reinterpret_cast<uint32_t*>(qcat + ((size_t)t * H + h) * (2 * DQ) + DL) + pr;
    dst[0] = bf16_half2(ra * smscale, rb * smscale, 0.f);
    dst[DQ / 2] = bf16_half2(ra * smscale, rb * smscale, 1.f);
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
                              const int32_t* cached_len, int n_new, int max_len, uint16_t* qcat,
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
                           const uint16_t* c_rope, const uint16_t* qcat,
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
