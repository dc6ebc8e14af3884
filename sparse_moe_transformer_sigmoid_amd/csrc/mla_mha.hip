// Kimi K2 multi-head latent attention for prompt-sized batches: the per-head
// form on gfx950.
//
// MLA ("Kimi K2 · Architecture", Fact sheet; "Kimi-K2-Base", Attention): per
// head the key is [W_uk c_j (128), k_rope_j (64)] and the value W_uv c_j
// (128), where c_j is position j's cached latent and W_uk, W_uv are the head's
// key and value rows of the key-value up-projection.  With many new tokens per
// sequence it is cheaper to form those keys and values once per position and
// head than to run every query through the 576-wide latent (the absorbed
// form of mla.hip):
//   per (query, position, head) the products cover 128 + 64 key features and
//   128 value features, against 576 + 512 latent features absorbed, and
//   expanding a position costs as much as about 150 queries attending to it.
// The results are the same function: q . k_j and sum_j p_j v_j are computed
// directly instead of through W_uk^T q and W_uv sum_j p_j c_j.
//
// Precision: keys, values, queries and probabilities are fp32 values; each is
// carried through the bf16 MFMA as its bf16 high part plus the bf16 rounding
// of the remainder, and a product takes the three terms hi*hi + hi*lo + lo*hi
// (the rotary keys are bf16 values, so their products take two), summed in
// fp32: within about 2^-16 of the fp32 product.
//
// 1. mla_kv_expand_kernel: for every visible position of every sequence and
//    head, K = W_uk c_j and V = W_uv c_j from the e4m3 codes (both exact in
//    bf16): per 128-latent block an MFMA sum, times (weight block scale x
//    cache scale), added in fp32; written as bf16 high and low halves, K
//    row-major and V transposed, in blocks of 32 positions.
// 2. mla_mha_kernel: flash-style causal attention per (sequence, head, 256
//    queries), eight waves of 32 queries; the step's 32 positions (both K
//    halves, the rotary keys, both V halves: 36 KiB) are copied straight into
//    one of three LDS stages two steps ahead; scores S^T = K Q^T, online
//    softmax per query, O^T += V^T P^T; the epilogue divides by the softmax
//    sum and writes each (token, head)'s 128 outputs as one 1x128 block of
//    the output projection's input (e4m3 codes + scale) and, optionally, in
//    fp32.
#include <math.h>

#include "k2_common.h"
#include "mla_common.h"
#include "mla_launch.h"

namespace k2 {

namespace {

constexpr int XB = 32;               // positions per expanded block and attention step
constexpr int XBLK = 4 * XB * DN;    // bf16 per block: K hi, K lo [32][128]; V hi, V lo [128][32]
constexpr int XP = 64;               // positions per expand workgroup

// eight e4m3 codes (two dwords, lowest byte first) -> eight bf16, exactly
__device__ __forceinline__ v8bf e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// v reduced over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of an
// MFMA result) by the maximum or the sum: two swaps of lane halves between two
// copies of v (VALU, no LDS traffic), each leaving v_l and its partner's value
// in the two results at every lane
template <bool MAX>
__device__ __forceinline__ float col_reduce(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = MAX ? fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]))
          : __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return MAX ? fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]))
             : __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// the sequence's cached length, clamped so that its n_new new positions stay
// inside the cache (the caller guarantees it; a bad value then gives wrong
// results, never an access outside the buffers)
__device__ __forceinline__ int cached_of(const int32_t* cached_len, int seq, int n_new,
                                         int max_len) {
  return min(max(cached_len[seq], 0), max_len - n_new);
}

// ------------------------------------------------------------ expansion
// Workgroup = (sequence, head, 64 positions), eight waves; wave w forms the
// keys (w < 4) or values (w >= 4) of features 32 (w % 4) .. + 31 for all 64
// positions.  The positions' codes (32 KiB) are copied once into LDS; each
// wave streams its 32 weight rows from global memory one 32-latent step
// ahead.  A 16x16x32 MFMA takes the weight rows as one operand and the codes
// of 16 positions as the other; keys are formed as K^T (lane: one position,
// 4 consecutive features), values as V (lane: one feature, 4 consecutive
// positions).  The workgroup's two blocks of keys and values (64 KiB) are
// assembled in LDS (rows padded so the 8-byte writes of 16 lanes fall on
// distinct banks) and then written as eight contiguous 8 KiB regions, every
// store a whole 16 bytes of a line.  Positions at or past the visible range
// are written as zeros (the attention masks them, and zero values keep
// p = 0 terms finite).
//
// Codes in LDS: position p's 16-byte chunk c at chunk slot c ^ (p % 16), so
// the 8-byte fragment reads of 16 consecutive positions at one latent offset
// fall on distinct banks.
constexpr int XW = 8;                  // waves per expand workgroup
constexpr int XF = 32;                 // features per wave
// LDS assembly of a workgroup's output: keys [block][hi, lo][32 positions][128
// features] with rows of 272 bytes, then values [block][hi, lo][128
// features][32 positions] with rows of 80 bytes; the codes share the start
constexpr int XK_LD = DN * 2 + 16, XV_LD = XB * 2 + 16;
constexpr int XK_BYTES = 2 * 2 * XB * XK_LD, XV_BYTES = 2 * 2 * DN * XV_LD;
constexpr int XS_BYTES = XK_BYTES + XV_BYTES;
static_assert(XS_BYTES >= XP * DL, "the assembly area holds the codes first");

template <bool VALUES>
__device__ __forceinline__ void expand_wave(int h, int p0, int valid, uint8_t* xs,
                                            const float* sc_s, const uint16_t* __restrict__ w,
                                            const float* __restrict__ sw, int f0, int lane) {
  const uint8_t* cl_s = xs;
  const int g = lane >> 4, l16 = lane & 15;
  const uint16_t* wrow = w + ((size_t)h * DN + f0 + l16) * DL + 8 * g;
  // B / A fragment of positions 16 pt + l16, latents k0 + 8 g .. + 7: bytes of
  // 16-byte chunk (k0 + 8 g) / 16, half g % 2 (k0 a multiple of 32)
  auto cfrag = [&](int pt, int k0) {
    const int p = 16 * pt + l16;
    const int c = (k0 >> 4) + (g >> 1);
    const uint2 c8 =
        *reinterpret_cast<const uint2*>(cl_s + p * DL + 16 * (c ^ l16) + 8 * (g & 1));
    return e4m3x8_bf16(c8.x, c8.y);
  };
  auto wfrag = [&](int ft, int k0) {
    return *reinterpret_cast<const v8bf*>(wrow + (size_t)16 * ft * DL + k0);
  };
  v4f acc[2][4];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[ft][pt] = v4f{0.f, 0.f, 0.f, 0.f};
  v8bf wc[2], wn[2];
  wc[0] = wfrag(0, 0);
  wc[1] = wfrag(1, 0);
#pragma unroll 1
  for (int b = 0; b < DL / QBLK; ++b) {
    v4f d[2][4];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) d[ft][pt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < QBLK / 32; ++kk) {
      const int k0 = b * QBLK + 32 * kk;
      if (k0 + 32 < DL) {
        wn[0] = wfrag(0, k0 + 32);
        wn[1] = wfrag(1, k0 + 32);
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const v8bf cf = cfrag(pt, k0);
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
          d[ft][pt] = VALUES ? mfma_bf16(cf, wc[ft], d[ft][pt]) : mfma_bf16(wc[ft], cf, d[ft][pt]);
      }
      if (k0 + 32 < DL) {
        wc[0] = wn[0];
        wc[1] = wn[1];
      }
    }
    const float s_w = sw[b];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if constexpr (VALUES) {
        // lane: feature f0 + 16 ft + l16, positions 16 pt + 4 g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = sc_s[(16 * pt + 4 * g + i) * (DL / QBLK) + b] * s_w;
#pragma unroll
          for (int ft = 0; ft < 2; ++ft) acc[ft][pt][i] += d[ft][pt][i] * sc;
        }
      } else {
        // lane: position 16 pt + l16, features f0 + 16 ft + 4 g + i
        const float sc = sc_s[(16 * pt + l16) * (DL / QBLK) + b] * s_w;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) acc[ft][pt] += d[ft][pt] * sc;
      }
    }
  }
  // every wave is done reading the codes before they are overwritten
  __syncthreads();
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    if constexpr (VALUES) {
      const int pl = 16 * pt + 4 * g;   // four positions, all in one block
      const int bi = pl / XB, r = pl % XB;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) {
        const int f = f0 + 16 * ft + l16;
        v4f v = acc[ft][pt];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (p0 + pl + i >= valid) v[i] = 0.f;
        uint8_t* row = xs + XK_BYTES + ((bi * 2) * DN + f) * XV_LD + 2 * r;
        *reinterpret_cast<uint2*>(row) =
            make_uint2(bf16_half2(v[0], v[1], 0.f), bf16_half2(v[2], v[3], 0.f));
        *reinterpret_cast<uint2*>(row + DN * XV_LD) =
            make_uint2(bf16_half2(v[0], v[1], 1.f), bf16_half2(v[2], v[3], 1.f));
      }
    } else {
      const int pl = 16 * pt + l16;
      const int bi = pl / XB, r = pl % XB;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) {
        const int f = f0 + 16 * ft + 4 * g;
        v4f v = acc[ft][pt];
        if (p0 + pl >= valid) v = v4f{0.f, 0.f, 0.f, 0.f};
        uint8_t* row = xs + ((bi * 2) * XB + r) * XK_LD + 2 * f;
        *reinterpret_cast<uint2*>(row) =
            make_uint2(bf16_half2(v[0], v[1], 0.f), bf16_half2(v[2], v[3], 0.f));
        *reinterpret_cast<uint2*>(row + XB * XK_LD) =
            make_uint2(bf16_half2(v[0], v[1], 1.f), bf16_half2(v[2], v[3], 1.f));
      }
    }
  }
}

// grid: S * H * (nblk / 2) workgroups of 512 threads; nblk = padded length / 32
// (even).  kv: per (sequence, head), nblk blocks of XBLK bf16.
__global__ __launch_bounds__(512, 4) void mla_kv_expand_kernel(
    int H, int n_new, int max_len, int nblk, const int32_t* __restrict__ cached_len,
    const uint8_t* __restrict__ c_codes, const float* __restrict__ c_scales,
    const uint16_t* __restrict__ uk, const uint16_t* __restrict__ uv,
    const float* __restrict__ s_kvb, uint16_t* __restrict__ kv) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[XS_BYTES];   // codes, then the output
  __shared__ float sc_s[XP * (DL / QBLK)];
  const int per = nblk / 2;
  const int sh = blockIdx.x / per, pb = blockIdx.x % per;
  const int seq = sh / H, h = sh % H;
  const int valid = cached_of(cached_len, seq, n_new, max_len) + n_new;
  const int p0 = pb * XP;
  if (p0 >= valid) return;   // never read: the attention stops at the last visible block
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* codes = c_codes + (size_t)seq * max_len * DL;
  // codes of positions p0 .. p0 + 63 (clamped to the visible range): wave w
  // copies positions 8 w .. 8 w + 7, two per instruction
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 8 * wave + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ (p & 15);
    lds_copy16(codes, (uint32_t)(min(p0 + p, valid - 1) * DL + 16 * c),
               lds_addr(xs + (8 * wave + 2 * i) * DL));
  }
  if (tid < XP * (DL / QBLK))
    sc_s[tid] = c_scales[((size_t)seq * max_len + min(p0 + tid / (DL / QBLK), valid - 1)) *
                             (DL / QBLK) + tid % (DL / QBLK)];
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __syncthreads();
  const float* sw = s_kvb + (size_t)(2 * h + (wave >> 2)) * (DL / QBLK);
  if (wave < 4)
    expand_wave<false>(h, p0, valid, xs, sc_s, uk, sw, XF * wave, lane);
  else
    expand_wave<true>(h, p0, valid, xs, sc_s, uv, sw, XF * (wave - 4), lane);
  __syncthreads();
  // the two blocks: K hi, K lo, V hi, V lo, each 8 KiB contiguous in kv
  uint16_t* dst0 = kv + ((size_t)sh * nblk + 2 * pb) * XBLK;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      uint8_t* dk = reinterpret_cast<uint8_t*>(dst0 + bi * XBLK + hl * XB * DN);
      const int kr = tid >> 4, kc = tid & 15;   // 32 rows x 16 chunks
      *reinterpret_cast<uint4*>(dk + kr * DN * 2 + 16 * kc) = *reinterpret_cast<const uint4*>(
          xs + ((bi * 2 + hl) * XB + kr) * XK_LD + 16 * kc);
      uint8_t* dv = reinterpret_cast<uint8_t*>(dst0 + bi * XBLK + (2 + hl) * XB * DN);
      const int vr = tid >> 2, vc = tid & 3;    // 128 rows x 4 chunks
      *reinterpret_cast<uint4*>(dv + vr * XB * 2 + 16 * vc) = *reinterpret_cast<const uint4*>(
          xs + XK_BYTES + ((bi * 2 + hl) * DN + vr) * XV_LD + 16 * vc);
    }
}

// ------------------------------------------------------------ attention
constexpr int MQ = 32;                   // queries per wave
constexpr int MW = 8;                    // waves per workgroup
constexpr int MQT = MQ * MW;             // queries per workgroup
constexpr int MNS = 3;                   // LDS stages (copies run two steps ahead)
constexpr float LAZY = 8.f;              // log2 margin before a query's reference maximum moves
// stage: K hi [32][256 B], K lo, V hi [128][64 B], V lo, rotary keys [32][128 B]
constexpr int ST_KL = XB * DN * 2, ST_VH = 2 * ST_KL, ST_VL = 3 * ST_KL, ST_KP = 4 * ST_KL;
constexpr int STAGE = ST_KP + XB * DR * 2;

struct MhaArgs {
  const float* q;             // [nsplit, T, H * 192] q_b projection K-slice partial sums
  const double* rot;          // [T, 32, 2] cosine and sine of each token's rotary angles
  const int32_t* cached_len;  // [S]
  const uint16_t* kv;         // expanded keys and values
  const uint16_t* c_rope;     // [S, max_len, 64] rotated keys (bf16)
  uint8_t* o_q;               // [T, H * 128] e4m3 codes
  float* o_s;                 // [T, H] their scales
  float* attn;                // [T, H * 128] fp32 or null
  int T, H, n_new, max_len, nblk, nq, nsplit, n_pairs;
  float smscale;
};

// Workgroup = (sequence, head, 256 consecutive new tokens); wave w: tokens
// 32 w .. + 31 of them as two 16-query tiles.  Copies and their LDS slots
// (chunk = 16 bytes): the A fragment of 16 positions (or features) reads one
// chunk of each of 16 rows, so each row's chunks are XOR-permuted to put
// those 16 reads on distinct banks; the copy of a row permutes the source
// chunks accordingly (direct-to-LDS copies write lane l at 16 l).
//   K row r (256 B): chunk c at slot c ^ (4 (r / 8) + r % 4)
//   rotary row r (128 B): chunk c at slot c ^ (2 (r / 8) + (r / 2) % 2)
//   V^T row f (64 B, 32 positions): chunk c at slot c ^ ((f / 4) % 4)
// Score tile pt (0, 1) of a step puts position 8 (i / 4) + 4 pt + i % 4 in
// its row i, so a lane's result rows 4 (l / 16) + i of both tiles are
// positions 8 (l / 16) .. + 7: exactly the eight K slots of lane l in the
// value MFMA, whose A operand (V^T) then reads one 16-byte chunk per row.
__global__ __launch_bounds__(512, 1) void mla_mha_kernel(const MhaArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t sl[MNS][STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  // XCD x (= block % 8) takes pairs x, x + 8, ...: first the last (heaviest)
  // query tile of each of them, then the tile before it, and so on, so that
  // the causal work of a tile shrinks as the launch drains
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int npx = (g.n_pairs + 7) / 8;   // pairs per XCD
  const int pair = (slot % npx) * 8 + x;
  if (pair >= g.n_pairs) return;
  const int qtile = g.nq - 1 - slot / npx;
  const int seq = pair / g.H, h = pair % g.H;
  const int cl = cached_of(g.cached_len, seq, g.n_new, g.max_len);
  const int valid = cl + g.n_new;
  const int q0 = qtile * MQT;
  const int nsteps = (cl + min(q0 + MQT, g.n_new) - 1) / XB + 1;
  const int wq0 = q0 + MQ * wave;
  const bool wact = wq0 < g.n_new;
  const int wsteps = wact ? (cl + min(wq0 + MQ, g.n_new) - 1) / XB + 1 : 0;
  const int wfull = (cl + wq0 + 1) / XB;   // steps every query of the wave sees whole

  // queries: lane holds query wq0 + 16 t2 + l16 (the last new token repeated
  // past n_new), features 32 ks + 8 gq .. + 7; rotary part rotated; scaled by
  // the softmax scale times log2 e, so the scores are in base-2 units and
  // p = 2^(s - max)
  v8bf qh[2][6], ql[2][6];
  int qpos[2];
  const size_t qld = (size_t)g.H * (DN + DR), slice = (size_t)g.T * qld;
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int qi = min(wq0 + 16 * t2 + l16, g.n_new - 1);
    qpos[t2] = cl + qi;
    const float* qp = g.q + (size_t)(seq * g.n_new + qi) * qld + h * (DN + DR) + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      float4 a = *reinterpret_cast<const float4*>(qp + 32 * ks);
      float4 b = *reinterpret_cast<const float4*>(qp + 32 * ks + 4);
      for (int s = 1; s < g.nsplit; ++s) {
        const float4 c = *reinterpret_cast<const float4*>(qp + s * slice + 32 * ks);
        const float4 d = *reinterpret_cast<const float4*>(qp + s * slice + 32 * ks + 4);
        a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
        b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
      }
      if (ks >= DN / 32) {
        // rotary pairs pr .. pr + 3 (the angles mla_latent_kernel formed for
        // this token's cache entry)
        const int pr = 16 * (ks - DN / 32) + 4 * gq;
        const double* cs = g.rot + ((size_t)(seq * g.n_new + qi) * (DR / 2) + pr) * 2;
        rope_apply(a.x, a.y, cs[0], cs[1], &a.x, &a.y);
        rope_apply(a.z, a.w, cs[2], cs[3], &a.z, &a.w);
        rope_apply(b.x, b.y, cs[4], cs[5], &b.x, &b.y);
        rope_apply(b.z, b.w, cs[6], cs[7], &b.z, &b.w);
      }
      const float m = g.smscale * 1.4426950408889634f;   // log2 e
      split8(make_float4(a.x * m, a.y * m, a.z * m, a.w * m),
             make_float4(b.x * m, b.y * m, b.z * m, b.w * m), &qh[t2][ks], &ql[t2][ks]);
    }
  }
  // every load above has returned before the first copy is issued: the copies'
  // waits below count only copies
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");

  const uint8_t* kvp = reinterpret_cast<const uint8_t*>(g.kv + (size_t)pair * g.nblk * XBLK);
  const uint8_t* rp = reinterpret_cast<const uint8_t*>(g.c_rope + (size_t)seq * g.max_len * DR);
  // copies of step j into stage st: wave w issues K hi, K lo, V hi and V lo
  // instruction w (4 K rows or 16 V rows each) and, waves 0-3, rotary
  // instruction w (8 rows)
  const int n_copies = wave < 4 ? 5 : 4;
  auto issue = [&](int st, int j) {
    uint8_t* sb = sl[st];
    const uint32_t bo = (uint32_t)j * (XBLK * 2);
    {
      const int r = 4 * wave + gq;
      const int c = l16 ^ (4 * (r >> 3) + (r & 3));
      const uint32_t src = bo + r * (DN * 2) + 16 * c;
      lds_copy16(kvp, src, lds_addr(sb + wave * 1024));
      lds_copy16(kvp, src + ST_KL, lds_addr(sb + ST_KL + wave * 1024));
    }
    {
      const int f = 16 * wave + (lane >> 2);
      const int c = (lane & 3) ^ ((f >> 2) & 3);
      const uint32_t src = bo + ST_VH + f * (XB * 2) + 16 * c;
      lds_copy16(kvp, src, lds_addr(sb + ST_VH + wave * 1024));
      lds_copy16(kvp, src + ST_KL, lds_addr(sb + ST_VL + wave * 1024));
    }
    if (wave < 4) {
      const int r = 8 * wave + (lane >> 3);
      const int c = (lane & 7) ^ (2 * (r >> 3) + ((r >> 1) & 1));
      const int p = min(j * XB + r, valid - 1);
      lds_copy16(rp, (uint32_t)(p * (DR * 2) + 16 * c), lds_addr(sb + ST_KP + wave * 1024));
    }
  };

  v4f o[2][DV / 16];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int ft = 0; ft < DV / 16; ++ft) o[t2][ft] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

  auto compute = [&](int st, int j) {
    const uint8_t* sb = sl[st];
    v4f s[2][2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) s[pt][t2] = v4f{0.f, 0.f, 0.f, 0.f};
    // twelve fragment groups per step: for each score tile pt, the four K
    // blocks (high and low halves), then the two rotary blocks; group u + 1's
    // fragments are read while group u's MFMAs run
    auto kload = [&](int u, v8bf& a, v8bf& b) {
      const int pt = u / 6, k = u % 6;
      const int r = 8 * (l16 >> 2) + 4 * pt + (l16 & 3);
      if (k < DN / 32) {
        const int o16 = r * (DN * 2) + 16 * ((4 * k + gq) ^ l16);
        a = *reinterpret_cast<const v8bf*>(sb + o16);
        b = *reinterpret_cast<const v8bf*>(sb + ST_KL + o16);
      } else {
        const int o16 = ST_KP + r * (DR * 2) + 16 * ((4 * (k - DN / 32) + gq) ^ (l16 >> 1));
        a = *reinterpret_cast<const v8bf*>(sb + o16);
      }
    };
    v8bf ca, cb, na, nb;
    kload(0, ca, cb);
#pragma unroll
    for (int u = 0; u < 12; ++u) {
      if (u + 1 < 12) kload(u + 1, na, nb);
      __builtin_amdgcn_sched_barrier(0);
      const int pt = u / 6, k = u % 6;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        s[pt][t2] = mfma_bf16(ca, qh[t2][k], s[pt][t2]);
        s[pt][t2] = mfma_bf16(ca, ql[t2][k], s[pt][t2]);
        if (k < DN / 32) s[pt][t2] = mfma_bf16(cb, qh[t2][k], s[pt][t2]);
      }
      if (u + 1 < 12) {
        ca = na;
        cb = nb;   // (a rotary group leaves b as it was; only K groups read it)
      }
    }
    // online softmax per query (lane: query 16 t2 + l16, positions
    // 32 j + 8 gq + 4 pt + i); the causal mask only on steps that reach past
    // some query of the wave
    v8bf ph[2], pl[2];
    if (j >= wfull) {
      const int kp0 = j * XB + 8 * gq;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kp0 + 4 * pt + i > qpos[t2]) s[pt][t2][i] = -INFINITY;
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      float v[8];
      float mx = -INFINITY;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[4 * pt + i] = s[pt][t2][i];
          mx = fmaxf(mx, v[4 * pt + i]);
        }
      // The reference maximum moves only when the step's maximum passes it by
      // more than LAZY (log2 units), so the probabilities stay below 2^LAZY
      // and the outputs are rarely rescaled; the normalisation by the sum
      // cancels the reference exactly.  Step 0 sees position 0, so every
      // query's reference is finite after it.
      const float mxq = col_reduce<true>(mx);
      const float mnew = mxq > mrun[t2] + LAZY ? mxq : mrun[t2];
      const float alpha = __builtin_amdgcn_exp2f(mrun[t2] - mnew);   // 1 where it did not move
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] = __builtin_amdgcn_exp2f(v[k] - mnew);
        sum += v[k];
      }
      lrun[t2] = lrun[t2] * alpha + sum;
      // the outputs are rescaled only when some query's reference moved
      if (__builtin_amdgcn_ballot_w64(mnew > mrun[t2]) != 0) {
#pragma unroll
        for (int ft = 0; ft < DV / 16; ++ft) o[t2][ft] *= alpha;
      }
      mrun[t2] = mnew;
      split8(make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7]), &ph[t2],
             &pl[t2]);
    }
    // O^T += V^T P^T (lane: query 16 t2 + l16, features 16 ft + 4 gq + i)
#pragma unroll
    for (int ft = 0; ft < DV / 16; ++ft) {
      const int o16 = (16 * ft + l16) * (XB * 2) + 16 * (gq ^ (l16 >> 2));
      const v8bf vh = *reinterpret_cast<const v8bf*>(sb + ST_VH + o16);
      const v8bf vl = *reinterpret_cast<const v8bf*>(sb + ST_VL + o16);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        o[t2][ft] = mfma_bf16(vh, ph[t2], o[t2][ft]);
        o[t2][ft] = mfma_bf16(vh, pl[t2], o[t2][ft]);
        o[t2][ft] = mfma_bf16(vl, ph[t2], o[t2][ft]);
      }
    }
  };

  issue(0, 0);
  if (nsteps > 1) issue(1, 1);
  for (int j = 0; j < nsteps; ++j) {
    // this wave's copies of step j are done once at most those of step j + 1
    // are outstanding; the barrier then publishes every wave's
    vm_wait(j + 1 < nsteps ? n_copies : 0);
    __syncthreads();
    // stage (j + 2) % 3 was last read in step j - 1, before this barrier
    if (j + 2 < nsteps) issue((j + 2) % MNS, j + 2);
    if (j < wsteps) compute(j % MNS, j);
  }
  if (!wact) return;

  // o / l, then the 1x128 block of each (token, head): e4m3 codes and scale
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const float l = col_reduce<false>(lrun[t2]);
    float amax = 0.f;
#pragma unroll
    for (int ft = 0; ft < DV / 16; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[t2][ft][i] = o[t2][ft][i] / l;
        amax = fmaxf(amax, fabsf(o[t2][ft][i]));
      }
    const float sc = fp8_scale(col_reduce<true>(amax));
    const int qi = wq0 + 16 * t2 + l16;
    if (qi >= g.n_new) continue;
    const size_t t = (size_t)seq * g.n_new + qi;
#pragma unroll
    for (int ft = 0; ft < DV / 16; ++ft) {
      const v4f v = o[t2][ft];
      const size_t e = t * g.H * DV + (size_t)h * DV + 16 * ft + 4 * gq;
      *reinterpret_cast<uint32_t*>(g.o_q + e) =
          cvt4_e4m3(clamp_fp8(v[0] / sc), clamp_fp8(v[1] / sc), clamp_fp8(v[2] / sc),
                    clamp_fp8(v[3] / sc));
      if (g.attn) *reinterpret_cast<float4*>(g.attn + e) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (gq == 0) g.o_s[t * g.H + h] = sc;
  }
}

}  // namespace

// ------------------------------------------------------------- launchers
int mla_mha_nblk(int max_len) { return (max_len + XP - 1) / XP * (XP / XB); }

size_t mla_mha_kv_bytes(int n_seq, int H, int max_len) {
  return (size_t)n_seq * H * mla_mha_nblk(max_len) * XBLK * 2;
}

hipError_t launch_mla_mha(int T, int H, int n_seq, int n_new, int max_len, int nsplit,
                          float smscale, const float* q, const double* rot,
                          const int32_t* cached_len, const uint8_t* c_codes,
                          const float* c_scales, const uint16_t* c_rope, const uint16_t* uk,
                          const uint16_t* uv, const float* s_kvb, uint16_t* kv, uint8_t* o_q,
                          float* o_s, float* attn, hipStream_t s) {
  if (n_seq <= 0 || n_new <= 0 || T != n_seq * n_new || n_new > max_len) return hipErrorInvalidValue;
  const int nblk = mla_mha_nblk(max_len);
  // the kernels address one (sequence, head)'s blocks, a sequence's codes and
  // its rotary keys with 32-bit byte offsets
  if ((size_t)nblk * XBLK * 2 > 0xFFFFFFFFu || (size_t)max_len * DL > 0xFFFFFFFFu)
    return hipErrorInvalidValue;
  mla_kv_expand_kernel<<<n_seq * H * (nblk / 2), XW * 64, 0, s>>>(
      H, n_new, max_len, nblk, cached_len, c_codes, c_scales, uk, uv, s_kvb, kv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MhaArgs a{};
  a.q = q;
  a.rot = rot;
  a.cached_len = cached_len;
  a.kv = kv;
  a.c_rope = c_rope;
  a.o_q = o_q;
  a.o_s = o_s;
  a.attn = attn;
  a.T = T;
  a.H = H;
  a.n_new = n_new;
  a.max_len = max_len;
  a.nblk = nblk;
  a.nq = (n_new + MQT - 1) / MQT;
  a.nsplit = nsplit;
  a.n_pairs = n_seq * H;
  a.smscale = smscale;
  const int grid = (a.n_pairs + 7) / 8 * 8 * a.nq;
  mla_mha_kernel<<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace k2
