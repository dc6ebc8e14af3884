// Grouped block-scaled FP8 GEMMs of the K2 experts on gfx950 MFMA.
//
// Experts are SwiGLU MLPs without biases ("Kimi-K2-Base", Feed-forward:
// down_proj(act_fn(gate_proj(x)) * up_proj(x)), act_fn = SiLU); weights are
// e4m3 with one fp32 scale per 128x128 block and activations e4m3 with one
// fp32 scale per token and 128 columns ("Kimi K2 · Architecture",
// config.json quantization_config).  Per 128-wide K block the MFMA sums
// exact e4m3 products into a fresh fp32 tile, which is then added to the
// running accumulator times (activation scale * weight scale).
//
// Work item = (group, 256-row weight chunk, m-tile of 16*TT rows).  A
// workgroup has 4 waves; wave w streams 64 weight rows (four 16x128 MFMA
// fragments per K block, 8 KiB, contiguous in the packed layout) straight
// into registers, double-buffered one K block ahead.  The m-tile's activation
// rows are gathered into LDS (double-buffered) as whole 128-byte lines, in an
// XOR-swizzled layout that keeps stores and fragment reads conflict-free.  MFMA:
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales, A = 16 weight rows,
// B = 16 tokens, so lane l of the 16x16 result holds weight rows
// 4*(l/16)..+3 of token l%16.
//
// Gate/up (GATEUP): the 256 rows of chunk j are hidden features
// 128j..128j+127 of gate and of up; wave w holds gate and up rows
// 32w..32w+31 of them, so silu(g)*u is formed in registers and the 1x128
// requantisation needs one cross-wave max.  Down: chunk j is output
// features 256j..256j+255; the epilogue optionally multiplies by the
// routing weight and writes fp32 rows.
//
// Workgroup ids are remapped so each XCD takes a contiguous run of work
// items: the m-tiles of one weight chunk, and the chunks of one expert, then
// share that XCD's L2.
#pragma once
#include <type_traits>

#include "k2_common.h"
#include "k2_launch.h"


namespace k2 {

namespace {

// largest K / 128 of either GEMM (d_model <= 16384, d_ff <= 65536)
constexpr int MAX_NKB = 512;

// work-item shares of even and odd XCDs in the 16-row (TT = 1) launches
constexpr int XCD_EVEN_SHARE = 15, XCD_ODD_SHARE = 13;

// workgroups that cover W <= grid items under the uneven split: 8 quotas of
// at most ceil(W * 15 / 112) each, for any W up to the even-split grid
inline int split_grid(int grid) {
  return (int)(((int64_t)grid * 2 * XCD_EVEN_SHARE / (XCD_EVEN_SHARE + XCD_ODD_SHARE) + 15) /
               8 * 8 + 8);
}

__device__ __forceinline__ v8i join8(v4i a, v4i b) {
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // atype = btype = 0 (e4m3), E8M0 scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

// Eight e4m3 codes (two dwords, lowest byte first) -> eight bf16, exactly:
// every e4m3 value, subnormals included, is a bf16 value.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int lo, int hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The same 16x16x128 e4m3 product as mfma_fp8, summed to fp32 precision:
// gfx950's FP8 MFMA adds its 128 products at reduced precision (about 11% of
// sums correctly rounded, errors up to 2^-15.6 of the sum of |products|, in
// an in-bounds probe), while the bf16 MFMA on the exactly converted codes
// rounds 99% of them correctly (worst 2^-24.9).  Instruction j takes bytes
// 8j..8j+7 of every lane's 32-byte fragment: the same K indices in A and B,
// so the four instructions cover each of the 128 products once.
__device__ __forceinline__ v4f mfma_fp8_exact(v8i a, v8i b) {
  v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[2 * j], a[2 * j + 1]),
                                                e4m3x8_to_bf16(b[2 * j], b[2 * j + 1]), d,
                                                0, 0, 0);
  return d;
}

// Direct global -> LDS loads (global_load_lds_dword / _dwordx4): lane l's
// 4 or 16 bytes from global [base + voff] land at LDS byte address
// M0 + l * size.  Completion is tracked by vmcnt like any vector load, in
// issue order; the compiler knows nothing of them (see BMODE).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_load16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

struct WorkItem {
  bool valid;
  bool shared_grp;
  int grp, nc, row0, mcount, ntt;
};

// Work item L (after the XCD remap) -> (group, weight chunk, m-tile).  The
// grid is a host-side upper bound; workgroups past the device-side m-tile
// count get valid = false.
//
// RE : RO is the share of work items an even : odd XCD gets.  Workgroups on
// odd-numbered XCDs run about 10% longer than on even ones (measured on every
// box, in both GEMMs), so the streaming (one m-tile per group) launches give
// even XCDs XCD_EVEN_SHARE items for every XCD_ODD_SHARE of an odd one, and
// all XCDs finish together; the grid must then hold 8 * ceil(quota_even)
// workgroups (see split_grid).
//
// BY16: the group's ceil(m / 16) token tiles are dealt out as evenly as
// possible over its m-tiles, the first ones taking one more (launches that
// skip the token tiles past a tile's rows: a group then executes
// 16 * ceil(m / 16) rows, and its m-tiles, which read the same weight
// chunks, take near-equal time and stay close together in L2); otherwise its
// rows are split into near-equal tiles.
template <int RE = 1, int RO = 1, bool BY16 = false>
__device__ __forceinline__ WorkItem decode_work(const GemmArgs& g, int BM) {
  WorkItem w{};
  const int Wtot = g.mt_start[g.G] * g.NC;
  const int b = blockIdx.x;
  w.valid = false;
  int L;
  if constexpr (RE == RO) {
    const int Wp = (Wtot + 7) & ~7;
    if (b >= Wp) return w;
    L = (b & 7) * (Wp >> 3) + (b >> 3);
  } else {
    // XCD x takes items [start_x, start_x + quota_x): pairs of (even, odd)
    // XCDs in order, quota qe for the even one and qo for the odd one
    const int x = b & 7, i = b >> 3;
    const int qe = (int)(((int64_t)Wtot * RE + 4 * (RE + RO) - 1) / (4 * (RE + RO)));
    const int qo = (int)(((int64_t)Wtot * RO + 4 * (RE + RO) - 1) / (4 * (RE + RO)));
    if (i >= ((x & 1) ? qo : qe)) return w;
    L = (x >> 1) * (qe + qo) + (x & 1) * qe + i;
  }
  if (L >= Wtot) return w;
  const int q = L / g.NC;
  const int lo = min(max(g.tile_group[q], 0), g.G - 1);   // mt_start[lo] <= q < mt_start[lo+1]
  w.grp = lo;
  w.shared_grp = lo >= g.E;
  int row0_g, m_g;
  if (w.shared_grp) {
    row0_g = g.P;
    m_g = g.T;
  } else {
    row0_g = min(max(g.offsets[lo], 0), g.P);
    m_g = min(max(g.offsets[lo + 1] - row0_g, 0), g.P - row0_g);
  }
  // the group's rows are split into ceil(m / BM) m-tiles of at most BM rows,
  // near-equal ones, so the last tile of a group is not mostly padding
  // (BY16: near-equal numbers of 16-row token tiles)
  const int mtiles = (m_g + BM - 1) / BM;
  const int rr = L - g.mt_start[lo] * g.NC;
  // order inside a group: blocks of up to SUPER m-tiles; within a block,
  // weight chunks outer and m-tiles inner, so a run of consecutive work items
  // (one XCD's L2) shares both the weight chunks and the activation tiles
  constexpr int SUPER = 8;
  const int blk = rr / (g.NC * SUPER);
  const int sm = min(SUPER, mtiles - blk * SUPER);        // m-tiles in this block
  const int r2 = rr - blk * g.NC * SUPER;
  w.nc = r2 / sm;
  const int mt = blk * SUPER + (r2 - w.nc * sm);
  int r_lo, r_hi;
  if constexpr (BY16) {
    const int n16 = (m_g + 15) >> 4, q16 = n16 / mtiles, x16 = n16 % mtiles;
    r_lo = 16 * (mt * q16 + min(mt, x16));
    r_hi = min(r_lo + 16 * (q16 + (mt < x16 ? 1 : 0)), m_g);
  } else {
    r_lo = (int)(((int64_t)mt * m_g) / mtiles);
    r_hi = (int)(((int64_t)(mt + 1) * m_g) / mtiles);
  }
  w.row0 = row0_g + r_lo;
  w.mcount = r_hi - r_lo;
  w.ntt = (w.mcount + 15) >> 4;
  w.valid = true;
  return w;
}

// activation row of the m-th row of a tile (padding rows repeat the last)
template <bool GATEUP>
__device__ __forceinline__ int act_row_of(const GemmArgs& g, const WorkItem& w, int m) {
  const int mm = min(m, w.mcount - 1);
  if constexpr (GATEUP) {
    if (w.shared_grp) return w.row0 + mm - g.P;
    const int tok = g.row_pair[w.row0 + mm] / g.k;
    return min(max(tok, 0), g.T - 1);
  } else {
    return w.row0 + mm;
  }
}

// Accumulators -> outputs.  acc[rt][tt] lane l holds weight rows
// 64 wave + 16 rt + 4 (l / 16) + r of token row 16 tt + l % 16.
// NTS: write the down rows with non-temporal stores (the launches that stream
// each weight chunk once; at larger tiles ordinary stores measure faster).
template <bool GATEUP, int TT, bool NTS>
__device__ __forceinline__ void epilogue(const GemmArgs& g, v4f (&acc)[4][TT], float* lds_red,
                                         const WorkItem& wi, int wave, int lane, int kslice) {
  const int nc = wi.nc, row0 = wi.row0, mcount = wi.mcount, ntt = wi.ntt;
  const bool shared_grp = wi.shared_grp;
  if constexpr (GATEUP) {
    // a = silu(g) * u for hidden 32w + 16h + 4(l/16) + r, h in {0,1}
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float mx = 0.f;
      if (tt < ntt) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = acc[h][tt][r], uv = acc[h + 2][tt][r];
            const float a = gv / (1.0f + expf(-gv)) * uv;
            acc[h][tt][r] = a;
            mx = fmaxf(mx, fabsf(a));
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (lane < 16) lds_red[(wave * TT + tt) * 16 + lane] = mx;
    }
    __syncthreads();
    const int nblk = g.I / QBLK;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < ntt) {
        const int j = lane & 15;
        float amax = lds_red[(0 * TT + tt) * 16 + j];
#pragma unroll
        for (int w = 1; w < 4; ++w) amax = fmaxf(amax, lds_red[(w * TT + tt) * 16 + j]);
        const float sc = fp8_scale(amax);
        const int m = tt * 16 + j;
        if (m < mcount) {
          const size_t row = (size_t)(row0 + m);
          uint8_t* dst = g.aq + row * g.I + nc * QBLK + 32 * wave + 4 * (lane >> 4);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const v4f a = acc[h][tt];
            const uint32_t q4 = cvt4_e4m3(clamp_fp8(a[0] / sc), clamp_fp8(a[1] / sc),
                                          clamp_fp8(a[2] / sc), clamp_fp8(a[3] / sc));
            *reinterpret_cast<uint32_t*>(dst + 16 * h) = q4;
          }
          if (wave == 0 && lane < 16) g.as[row * nblk + nc] = sc;
        }
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < ntt) {
        const int m = tt * 16 + (lane & 15);
        if (m < mcount) {
          const int row = row0 + m;
          if (g.out_bf16) {
            // out = bf16(res + row), the residual add of a dense projection
            const size_t o0 = (size_t)row * g.d + nc * 256 + 64 * wave + 4 * (lane >> 4);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              const v4f o = acc[rt][tt];
              const uint2 xr = *reinterpret_cast<const uint2*>(g.res + o0 + 16 * rt);
              const uint32_t w0 = f32_to_bf16_rne(bf16_to_f32(xr.x & 0xFFFFu) + o[0]) |
                                  (f32_to_bf16_rne(bf16_to_f32(xr.x >> 16) + o[1]) << 16);
              const uint32_t w1 = f32_to_bf16_rne(bf16_to_f32(xr.y & 0xFFFFu) + o[2]) |
                                  (f32_to_bf16_rne(bf16_to_f32(xr.y >> 16) + o[3]) << 16);
              *reinterpret_cast<uint2*>(g.out_bf16 + o0 + 16 * rt) = make_uint2(w0, w1);
            }
            continue;
          }
          float wt = 1.f;
          const bool mul = g.weighted && !shared_grp;
          if (mul) wt = g.topk_w[min(max(g.row_pair[row], 0), g.P - 1)];
          // split-K launches write one [P, d] slice of partial sums per K slice
          float* dst = shared_grp ? g.shared_out + (size_t)(row - g.P) * g.d
                                  : g.rows + ((size_t)kslice * g.P + row) * g.d;
          dst += nc * 256 + 64 * wave + 4 * (lane >> 4);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            v4f o = acc[rt][tt];
            if (mul) o = o * wt;
            if constexpr (NTS)
              __builtin_nontemporal_store(o, reinterpret_cast<v4f*>(dst + 16 * rt));
            else
              *reinterpret_cast<float4*>(dst + 16 * rt) = make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  }
}

// TT: 16-row token tiles per m-tile; NBUF: weight register ring depth (prefetch
// distance NBUF-1 K blocks); NT: stream weights with non-temporal loads, for
// launches where each weight chunk is read by a single m-tile.
// BSETS: activation register sets (2: loaded two K blocks ahead; 1: one block
// ahead, saving registers); MINW: waves per SIMD the register budget must allow.
// GRPX: token tiles per scheduling group (0: the default for TT and MINW).
// BMODE: activation staging.  0: through BSETS register sets, stored to LDS
// at the end of each step.  1: loaded straight into LDS (no staging
// registers) and each token tile's B fragment read one tile ahead.
// ILV (BMODE 0): if nonzero, the issue order inside a scheduling group is
// fixed: its LDS reads, two MFMAs, then each further MFMA after ILV VALU
// instructions (the promotion FMAs of the MFMA two back).
// EXACT (BMODE 0): each 128-wide block product is summed by mfma_fp8_exact
// (twice the MFMA cycles), so the gate/up values the requantisation decides
// on are correct to fp32 rounding; for launches that wait on HBM, not MFMA.
// SPLITK (down form): the K blocks are cut into gridDim.y equal slices, slice
// blockIdx.y writing its partial sums to its own [P, d] slice of `rows`
// (for small batches, whose few work items would not fill the chip).
template <bool GATEUP, int TT, int NBUF, bool NT, int BSETS = 2, int MINW = 1, int GRPX = 0,
          int BMODE = 0, int ILV = 0, bool EXACT = false, bool SPLITK = false>
__global__ __launch_bounds__(256, MINW) void gemm_fp8_kernel(const GemmArgs g) {
  static_assert(NBUF >= 2 && NBUF <= 4, "NBUF must be 2, 3 or 4");
  static_assert(BSETS == 1 || BSETS == 2, "BSETS must be 1 or 2");
  // BMODE 1 ends each step with a wait that counts the 8 weight loads of one
  // ring slot issued after the step's direct loads (one slot per step)
  static_assert(BMODE == 0 || (BMODE == 1 && NBUF == 2), "BMODE 1 needs NBUF 2");
  static_assert(!EXACT || (BMODE == 0 && ILV == 0), "EXACT is implemented for BMODE 0 only");
  static_assert(!SPLITK || !GATEUP, "SPLITK is implemented for the down form only");
  constexpr int BM = 16 * TT;
  // 128-row tiles compute only their token tiles that hold rows: the K loop
  // is instantiated for 1 .. 8 active tiles and chosen once per workgroup
  // (a branch inside the loop costs the register allocation dearly); the
  // group's token tiles are dealt out evenly over its m-tiles
  constexpr bool SKIP = TT == 8;
  constexpr int CPT = (TT * 128 + 255) / 256;   // 16-byte staging chunks per thread
  // LDS rows past the tile (TT < 2) are write-only padding: every thread
  // stages its chunk unconditionally, keeping the K loop free of branches
  constexpr int LDS_B = (TT * 2048 > 256 * 16 * ((TT * 128 + 255) / 256)) ? TT * 2048
                                                                          : 256 * 16 * ((TT * 128 + 255) / 256);
  // LDS double buffers of the activation tiles and their scales (the buffer
  // of each step is a compile-time choice in the unrolled K loop)
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[LDS_B], lds_b1[LDS_B];
  __shared__ float lds_sa0[256], lds_sa1[256];
  auto lds_b = [&](int buf) -> uint8_t* { return buf ? lds_b1 : lds_b0; };
  auto lds_sa = [&](int buf) -> float* { return buf ? lds_sa1 : lds_sa0; };
  // this chunk's weight scales for every K block, loaded once: scalar loads in
  // the loop would share lgkmcnt with the LDS reads and stall each step on
  // a memory round trip
  __shared__ float lds_sw[2 * MAX_NKB];
  __shared__ float lds_red[GATEUP ? 4 * TT * 16 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const WorkItem wi = TT == 1 ? decode_work<XCD_EVEN_SHARE, XCD_ODD_SHARE>(g, BM)
                              : decode_work<1, 1, SKIP>(g, BM);
  if (!wi.valid) return;
  const int grp = wi.grp, nc = wi.nc, row0 = wi.row0, mcount = wi.mcount;
  const int ntt = __builtin_amdgcn_readfirstlane(wi.ntt);
  // K slice of this workgroup: blocks kbs .. kbs + nkb_s - 1
  const int kslice = SPLITK ? (int)blockIdx.y : 0;
  const int nkb_s = SPLITK ? g.nkb / (int)gridDim.y : g.nkb;
  const int kbs = kslice * nkb_s;
  const uint8_t* const actp = g.act + (size_t)kbs * 128;
  const bool shared_grp = wi.shared_grp;

  auto act_row = [&](int m) { return act_row_of<GATEUP>(g, wi, m); };

  // Activation tiles in LDS: row j of token tile t at byte 2048 t + 128 j, its 16-byte
  // chunk c (columns 16c..16c+15) at position c ^ ((j / 2) % 8) of the row.
  // Thread (wave w, lane l) stages, in instruction i, 16 bytes of tile row
  // 32 i + 8 w + l / 8 into LDS chunk 256 i + 64 w + l (the destination
  // that direct-to-LDS loads require: lane l of a wave's instruction lands
  // at 16 l), which under the swizzle is chunk (l % 8) ^ (4 (w % 2) + l / 16)
  // of that row.  Every load instruction thus reads 8 whole 128-byte lines.
  // Stores (8 rows x 8 positions per wave) and fragment reads (16 rows, one
  // chunk each) both hit 16 distinct positions modulo 256 bytes.
  uint32_t boff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    // tid / 8 = 8 w + l / 8 and (tid / 16) % 8 = 4 (w % 2) + l / 16
    const int r = 32 * i + (tid >> 3);   // past the tile: clamped row
    const int c = (tid & 7) ^ ((tid >> 4) & 7);
    boff[i] = (uint32_t)act_row(r) * (uint32_t)g.act_ld + 16 * c;
  }
  // byte offsets, within a token tile, of this lane's two 16-byte halves of
  // its B fragment (token row lane % 16, columns 32 (lane / 16) + 16 p)
  const int bj = lane & 15, bsw = (bj >> 1) & 7;
  const uint32_t brd0 = 128u * bj + 16u * ((2 * (lane >> 4)) ^ bsw);
  const uint32_t brd1 = 128u * bj + 16u * ((2 * (lane >> 4) + 1) ^ bsw);
  // thread tid stages the activation scale of tile row tid (clamped past the tile)
  const uint32_t saoff = (uint32_t)act_row(tid) * g.nkb + kbs;

  // wave-uniform base of this wave's weight rows; per-lane 32-bit offsets
  // (the wave's rows span nkb * 8 KiB <= 4 MiB), so loads take the
  // scalar-base + vector-offset form and no 64-bit address registers
  const uint8_t* wp = g.wpk + (size_t)grp * g.expert_stride +
                      (size_t)(nc * 4 + wave) * (size_t)g.nkb * 8192 + (size_t)kbs * 8192;
  const uint32_t wlane = lane * 16;
  const float* swp_base = g.wscale + (size_t)grp * g.wscale_stride + (size_t)nc * g.nkb * 2;

  // gate/up: [kb][gate, up] of chunk nc; down: [row block 2nc + h][kb], h = 0, 1
  for (int i = tid; i < 2 * g.nkb; i += 256) lds_sw[i] = swp_base[i];

  // accumulators: zeroed, accumulated and written out inside each K-loop
  // instance, so no value of them is live where the instances meet
  v4f acc[4][TT];

  // weight fragments: a ring of NBUF register buffers, loaded NBUF-1 K blocks ahead;
  // activations: two register sets, loaded two K blocks ahead, stored to LDS one
  // block ahead (LDS double buffer)
  v8i wbuf[NBUF][4];
  v4i breg[BSETS][CPT];
  float sareg[2] = {0.f, 0.f};

  // ntc: std::true_type for non-temporal weight loads
  auto load_w = [&](v8i (&w)[4], int kb, auto ntc) {
    const uint8_t* p = wp + (uint32_t)(wlane + kb * 8192);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const v4i* p4 = reinterpret_cast<const v4i*>(p + rt * 2048);
      if constexpr (decltype(ntc)::value) {
        w[rt] = join8(__builtin_nontemporal_load(p4), __builtin_nontemporal_load(p4 + 64));
      } else {
        w[rt] = join8(p4[0], p4[64]);
      }
    }
  };
  auto load_b = [&](int set, int kb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      breg[set][i] = *reinterpret_cast<const v4i*>(actp + (uint32_t)(boff[i] + kb * 128));
    sareg[set] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(g.act_s) +
                                                 (uint32_t)((saoff + kb) * 4));
  };
  // BMODE 1: activation tiles go straight from global memory into LDS
  // (global_load_lds, no staging registers).  They are issued from inline
  // assembly: the compiler inserts no waits for them (its own tracking of
  // such loads waits for every outstanding load, the weight prefetch
  // included), and the step that issues them ends with an explicit wait and
  // barrier.  Byte offsets are 32-bit: rows * act_ld < 2^32.
  auto dma_b = [&](int buf, int kb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      lds_load16(actp, boff[i] + kb * 128, lds_addr(&lds_b(buf)[(256 * i + 64 * wave) * 16]));
    lds_load4(g.act_s, (saoff + kb) * 4, lds_addr(&lds_sa(buf)[64 * wave]));
  };
  auto store_b = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<v4i*>(&lds_b(buf)[(tid + 256 * i) * 16]) = breg[set][i];
    lds_sa(buf)[tid] = sareg[set];
  };
  auto weight_scales = [&](int kb, float& s_gate_or_down, float& s_up) {
    if constexpr (GATEUP) {
      s_gate_or_down = lds_sw[2 * (kb + kbs)];
      s_up = lds_sw[2 * (kb + kbs) + 1];
    } else {
      s_gate_or_down = lds_sw[(wave >> 1) * g.nkb + kb + kbs];
      s_up = s_gate_or_down;
    }
  };
  // Every tile of the m-tile is computed (rows past mcount are discarded at
  // the end): no branches in the hot loop, so the MFMA of one tile overlaps
  // the fp32 scaling of the previous tile's result.  Token tiles go in groups
  // of GRP; a scheduling fence between groups keeps the compiler from hoisting
  // every B fragment at once (register pressure at large TT; one tile per
  // group when the register budget is sized for 2 waves/SIMD).
  constexpr int GRP = GRPX ? GRPX : (TT < 4 ? TT : (MINW > 1 ? 1 : 4));
  // BMODE 1: one token tile at a time, the next tile's B fragment and scale
  // read from LDS before the current tile's MFMAs (its latency hides behind
  // them), promotion FMAs one MFMA behind
  auto compute_la = [&](const v8i (&w)[4], int buf, int kb, auto na) {
    constexpr int NA = decltype(na)::value;
    float swg, swu;
    weight_scales(kb, swg, swu);
    auto read_b = [&](int t, v8i& b, float& sa) {
      const uint8_t* bp = &lds_b(buf)[t * 2048];
      b = join8(*reinterpret_cast<const v4i*>(bp + brd0), *reinterpret_cast<const v4i*>(bp + brd1));
      sa = lds_sa(buf)[t * 16 + (lane & 15)];
    };
    v8i bc;
    float sac;
    read_b(0, bc, sac);
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      v8i bn = bc;
      float san = sac;
      if (t + 1 < NA) read_b(t + 1, bn, san);
      const float s0 = sac * swg, s1 = sac * swu;
      v4f prev = mfma_fp8(w[0], bc);
#pragma unroll
      for (int rt = 1; rt < 4; ++rt) {
        const v4f cur = mfma_fp8(w[rt], bc);
        acc[rt - 1][t] += prev * (rt - 1 < 2 ? s0 : s1);
        prev = cur;
      }
      acc[3][t] += prev * s1;
      bc = bn;
      sac = san;
      if (t + 1 < NA) __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute = [&](const v8i (&w)[4], int buf, int kb, auto na) {
    constexpr int NA = decltype(na)::value;
    static_assert(NA == TT || GRP == 1, "partial tiles need one token tile per group");
    if constexpr (BMODE == 1) {
      compute_la(w, buf, kb, na);
      return;
    }
    float swg, swu;
    weight_scales(kb, swg, swu);
#pragma unroll
    for (int t0 = 0; t0 < NA; t0 += GRP) {
      v8i bf[GRP];
      float s0[GRP], s1[GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const uint8_t* bp = &lds_b(buf)[(t0 + u) * 2048];
        bf[u] = join8(*reinterpret_cast<const v4i*>(bp + brd0),
                      *reinterpret_cast<const v4i*>(bp + brd1));
        const float sa_t = lds_sa(buf)[(t0 + u) * 16 + (lane & 15)];
        s0[u] = sa_t * swg;
        s1[u] = sa_t * swu;
      }
      auto mm = [](const v8i& a, const v8i& b) {
        if constexpr (EXACT) return mfma_fp8_exact(a, b);
        else return mfma_fp8(a, b);
      };
      v4f prev = mm(w[0], bf[0]);
#pragma unroll
      for (int i = 1; i < 4 * GRP; ++i) {
        const int u = i >> 2, rt = i & 3;
        const v4f cur = mm(w[rt], bf[u]);
        const int pu = (i - 1) >> 2, pr = (i - 1) & 3;
        acc[pr][t0 + pu] += prev * (pr < 2 ? s0[pu] : s1[pu]);
        prev = cur;
      }
      acc[3][t0 + GRP - 1] += prev * s1[GRP - 1];
      if constexpr (ILV) {
        // issue order inside the group: its LDS reads, two MFMAs, then each
        // further MFMA after ILV VALU instructions (the four promotion FMAs
        // of the MFMA two back, and a scale product)
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * GRP, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int i = 2; i < 4 * GRP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, ILV, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 8 + 2 * GRP, 0);
      }
      if (t0 + GRP < NA) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---------------------------------------------------------------- K loop
  // Block kb: weights in wbuf[kb % NBUF] with scales sw[kb % NBUF]; activations
  // in LDS buffer kb & 1, staged from register set (kb & 1) (BMODE 0) or
  // loaded there directly (BMODE 1).  Vector loads retire in issue order, so
  // each step issues the activations before the weights of block
  // kb+NBUF-1, and ends by waiting only for the activations (BMODE 0: those
  // of block kb+1, issued one step earlier).
  auto kloop = [&](auto ntc, auto na) {
  const int nkb = nkb_s;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (BMODE == 1) {
    dma_b(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // block 0, before the barrier below
  } else {
    // kb0 = 0, through an asm the compiler cannot see into and whose text
    // differs per instance: the instances' first loads are then not merged
    // ahead of the branch that picks one (their registers would stay live
    // through the other instances)
    int kb0;
    asm volatile("s_mov_b32 %0, 0 ; active tiles %1" : "=s"(kb0) : "i"(decltype(na)::value));
    load_b(0, kb0);
    if (BSETS == 2 && nkb > 1) load_b(BSETS - 1, kb0 + 1);
  }
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < nkb) load_w(wbuf[i], i, ntc);
  if constexpr (BMODE != 1) store_b(0, 0);
  __syncthreads();
  // One step: prefetch (activations of kb+2, weights of kb+NBUF-1; indices
  // clamped to the last block, so the tail re-reads a block instead of
  // branching), compute block kb, stage block kb+1 into LDS, barrier.  STEP is
  // a multiple of NBUF and of 2, so every buffer index is a compile-time
  // constant; full STEPs run without guards, the tail with them (BMODE 1:
  // one loop, the later steps of each STEP guarded).
  constexpr int STEP = (NBUF & 1) ? 2 * NBUF : NBUF;
  auto step = [&](const int j, const int kb) {
    const int cur = j & 1;
    if constexpr (BMODE == 1) {
      // LDS buffer cur ^ 1 was last read in the previous step, before its barrier
      dma_b(cur ^ 1, min(kb + 1, nkb - 1));
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (BSETS == 2) {
      load_b(cur, min(kb + 2, nkb - 1));
    } else {
      load_b(0, min(kb + 1, nkb - 1));
    }
    load_w(wbuf[(j + NBUF - 1) % NBUF], min(kb + NBUF - 1, nkb - 1), ntc);
    // keep the prefetches issued here: the scheduler would otherwise sink
    // them next to their use to save registers, undoing the ring
    __builtin_amdgcn_sched_barrier(0);
    compute(wbuf[j % NBUF], cur, kb, na);
    if constexpr (BMODE == 1) {
      // This wave's direct loads of block kb+1 are older than the 8 weight
      // loads issued after them, so vmcnt(8) completes them without waiting
      // for those weights (a barrier with a release fence would wait for
      // every load); then the barrier publishes block kb+1 to all waves.
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" : : : "memory");
    } else {
      store_b(BSETS == 2 ? cur ^ 1 : 0, cur ^ 1);
      __syncthreads();
    }
  };
  if constexpr (BMODE == 1) {
    // one loop with a uniform guard on the later steps of a STEP: a separate
    // tail would keep the prologue's weight block alive across the loop (for
    // the case of no full STEP), which spills at this register budget
    for (int kb0 = 0; kb0 < nkb; kb0 += STEP) {
#pragma unroll
      for (int j = 0; j < STEP; ++j)
        if (j == 0 || kb0 + j < nkb) step(j, kb0 + j);
    }
  } else {
    int kb0 = 0;
    for (; kb0 + STEP <= nkb; kb0 += STEP) {
#pragma unroll
      for (int j = 0; j < STEP; ++j) step(j, kb0 + j);
    }
#pragma unroll
    for (int j = 0; j < STEP; ++j)
      if (kb0 + j < nkb) step(j, kb0 + j);
  }
  epilogue<GATEUP, TT, NT>(g, acc, lds_red, wi, wave, lane, kslice);
  };
  // The shared expert's group has several m-tiles in the launches whose
  // routed groups have one: its weight chunks are read once per m-tile, so
  // that group loads them through L2 while routed chunks stream past it.
  using all_tiles = std::integral_constant<int, TT>;
  if constexpr (NT) {
    if (wi.shared_grp) kloop(std::false_type{}, all_tiles{});
    else kloop(std::true_type{}, all_tiles{});
  } else if constexpr (SKIP) {
    switch (ntt) {
      case 1: kloop(std::false_type{}, std::integral_constant<int, 1>{}); break;
      case 2: kloop(std::false_type{}, std::integral_constant<int, 2>{}); break;
      case 3: kloop(std::false_type{}, std::integral_constant<int, 3>{}); break;
      case 4: kloop(std::false_type{}, std::integral_constant<int, 4>{}); break;
      case 5: kloop(std::false_type{}, std::integral_constant<int, 5>{}); break;
      case 6: kloop(std::false_type{}, std::integral_constant<int, 6>{}); break;
      case 7: kloop(std::false_type{}, std::integral_constant<int, 7>{}); break;
      default: kloop(std::false_type{}, all_tiles{}); break;
    }
  } else {
    kloop(std::false_type{}, all_tiles{});
  }
}

}  // namespace

// gate/up launch of 128-row m-tiles (compiled in its own translation unit)
hipError_t launch_gateup_tt8(const GemmArgs& a, int grid, hipStream_t s);

}  // namespace k2
