// One training step of the K2 MoE layer on gfx950: the forward in BF16
// compute that keeps FP8 copies of the up-projection and SwiGLU inputs, and
// the backward that reads them.
//
// "Kimi-K2-Base", Pretraining recipe, Training precision: no FP8 in
// computation; the inputs of the MoE up-projections and of SwiGLU are stored
// as FP8-E4M3 in 1x128 tiles with FP32 scales.  Here h = RMSNorm(x) (the
// input of the gate/up projections and of the router) is stored as the
// 1x128 codes the inference path already makes of it, and g, u (the gate and
// up outputs, SwiGLU's inputs) as 1x128 codes along the hidden dimension of
// each row.  Every GEMM is bf16 x bf16 with fp32 accumulation
// (v_mfma_f32_16x16x32_bf16); the backward recomputes a = silu(g) u from the
// stored g, u.
//
// One GEMM template covers the four row-tiled products of the step:
//   forward gate/up   C[2I rows of W_gate, W_up][rows]  = W h^T      (+ SwiGLU, FP8 copies)
//   forward down      C[d][rows]                        = W_down a^T (+ routing weight)
//   dgrad down        C[I][rows]                        = W_down^T dy^T (+ dw, dg, du)
//   dgrad gate/up     C[d][rows]                        = [W_gate; W_up]^T [dg; du]^T
// and train_wgrad_kernel the weight gradients
//   wgrad             C[out][in]  = sum over a group's rows of X^T Y
// (both operands K-blocked transposed copies).  A workgroup computes a 256 x
// 128 tile (4 waves of 64 M rows, 8 16-row N tiles); each wave streams its A
// rows straight into registers one K step ahead, the 128 B rows are staged
// through LDS (double-buffered), and lane l of a 16x16 result holds M rows
// 4(l/16)..+3 of N column l%16.
#include <math.h>

#include <algorithm>

#include "k2_common.h"
#include "k2_launch.h"
#include "train_launch.h"

namespace k2 {

namespace {

constexpr int TK = 32;       // K per MFMA, per wgrad step and per K block of the blocked layouts
constexpr int TKR = 64;      // K per step of the row-tiled products (each A row's 128-byte line
                             // is read whole, as two 16-byte halves per lane)
constexpr int BR_LD = TKR + 8;   // bf16 stride of a staged row-tiled B row (144 bytes)
constexpr int TN = 128;      // N per workgroup (rows of a group, or input features)
constexpr int TMW = 64;      // M rows per wave
constexpr int B_LD = TK + 8;  // bf16 stride of a staged B row (80 bytes: conflict-free)
constexpr int SUPER = 8;     // m-tiles per scheduling block inside a group (L2 reuse)

__device__ __forceinline__ v4f mfma16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

// e4m3 code byte i (a compile-time index after unrolling) of word w -> float (exact)
__device__ __forceinline__ float e4m3_byte(uint32_t w, int i) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f p = i >= 2 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                       : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return (i & 1) ? p[1] : p[0];
}

struct TileWork {
  bool valid;
  int grp, nc, row0, mcount;   // rows: [row0, row0 + mcount) of the permuted order
  int mi, ni;                  // wgrad: M and N tile
};

// Work item of the row-tiled modes: (group, 256-row M chunk, tile of up to
// 128 rows), the rows of a group dealt out evenly in 16-row units.  The
// grid is a host upper bound; items past the device count exit.
__device__ __forceinline__ TileWork decode_rows(const TrainGemmArgs& g) {
  TileWork w{};
  const int Wtot = g.mt_start[g.G] * g.NC;
  const int b = blockIdx.x;
  const int Wp = (Wtot + 7) & ~7;
  if (b >= Wp) return w;
  const int L = (b & 7) * (Wp >> 3) + (b >> 3);   // each XCD takes a contiguous run
  if (L >= Wtot) return w;
  const int q = L / g.NC;
  const int grp = min(max(g.tile_group[q], 0), g.G - 1);
  int r0, m;
  if (grp >= g.E) {
    r0 = g.P;
    m = g.T;
  } else {
    r0 = min(max(g.offsets[grp], 0), g.P);
    m = min(max(g.offsets[grp + 1] - r0, 0), g.P - r0);
  }
  const int mtiles = (m + TN - 1) / TN;
  if (mtiles == 0) return w;
  const int rr = L - g.mt_start[grp] * g.NC;
  const int blk = rr / (g.NC * SUPER);
  const int sm = min(SUPER, mtiles - blk * SUPER);
  const int r2 = rr - blk * g.NC * SUPER;
  w.nc = r2 / sm;
  const int mt = blk * SUPER + (r2 - w.nc * sm);
  const int n16 = (m + 15) >> 4, q16 = n16 / mtiles, x16 = n16 % mtiles;
  const int lo = 16 * (mt * q16 + min(mt, x16));
  const int hi = min(lo + 16 * (q16 + (mt < x16 ? 1 : 0)), m);
  w.grp = grp;
  w.row0 = r0 + lo;
  w.mcount = hi - lo;
  w.valid = w.mcount > 0 && w.nc < g.NC;
  return w;
}

// Work item of the weight gradients: (group, WGRAD_M-row M tile, 128-column N
// tile).  An item's K is its group's rows, so the shared expert's items (T
// rows each, groups E .. G-1) are about T / (rows per routed expert) times as
// long as a routed one.  Every XCD (workgroup b runs on XCD b mod 8) starts
// with an equal share of the shared items -- shared item j on XCD j mod 8,
// longest work first -- and then takes a contiguous run of routed items, in
// which the M tiles of one N tile are adjacent (they share that N tile's Y
// rows in the XCD's L2).
__device__ __forceinline__ TileWork decode_wgrad(const TrainGemmArgs& g) {
  TileWork w{};
  const int per = g.MT * g.NT;
  const int Wtot = g.G * per;
  const int b = blockIdx.x;
  const int Wp = (Wtot + 7) & ~7;
  if (b >= Wp) return w;
  const int x = b & 7, i = b >> 3, slots = Wp >> 3;
  const int R = min(g.E, g.G) * per;   // routed items
  const int S = Wtot - R;              // shared items
  const int sq = S >> 3, sr = S & 7;
  const int sh_x = sq + (x < sr ? 1 : 0);   // shared items of XCD x
  int L;
  if (i < sh_x) {
    L = R + x + 8 * i;
  } else {
    // XCD x's routed run follows those of XCDs 0 .. x-1
    L = x * slots - (sq * x + min(x, sr)) + (i - sh_x);
    if (L >= R) return w;
  }
  w.grp = L / per;
  const int rr = L - w.grp * per;
  // M tiles inner: the items sharing an input-feature tile of Y run together
  w.ni = rr / g.MT;
  w.mi = rr - w.ni * g.MT;
  w.valid = true;
  return w;
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void train_gemm_kernel(const TrainGemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][TN * BR_LD];
  __shared__ float red[4 * 8 * 16 * 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;

  static_assert(MODE != TM_WGRAD, "weight gradients use train_wgrad_kernel");
  constexpr bool KBLK_A = MODE == TM_BWD_DOWN || MODE == TM_BWD_GU;
  const TileWork wi = decode_rows(g);
  if (!wi.valid) return;
  const int grp = wi.grp;

  // ---- operand row pointers
  const int nks = g.K / TKR;   // K steps
  const uint16_t* arow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* base;
    size_t row;
    if constexpr (MODE == TM_FWD_GU) {
      base = (mt < 2 ? g.A : g.A2) + (size_t)grp * g.a_stride;
      row = (size_t)(128 * wi.nc + 32 * wave + 16 * (mt & 1) + l16);
    } else {
      base = g.A + (size_t)grp * g.a_stride;
      row = (size_t)(256 * wi.nc + TMW * wave + 16 * mt + l16);
    }
    // dgrad: A is a K-blocked transposed weight copy, step s of row r at
    // s * lda + 32 r (lda = rows * 32); otherwise row-major with stride lda
    arow[mt] = base + row * (size_t)(KBLK_A ? TK : g.lda) + 8 * q4;
  }
  // B rows staged by this thread: tile rows tid/4 and tid/4 + 64, K chunks
  // (tid % 4) and (tid % 4) + 4 of 8 each
  const uint16_t* brow[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int tr = (tid >> 2) + 64 * c;
    size_t src;
    const int r = wi.row0 + min(tr, wi.mcount - 1);   // rows past the tile repeat the last
    if constexpr (MODE == TM_FWD_GU || MODE == TM_BWD_DOWN) {
      int tok = r >= g.P ? r - g.P : g.row_pair[r] / g.k;
      tok = min(max(tok, 0), g.T - 1);
      src = (size_t)tok * g.ldb;
    } else {
      src = (size_t)r * g.ldb;
    }
    brow[c] = g.B + src + 8 * (tid & 3);
  }

  v4f acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  // A: K halves kh = 0, 1 of a step (32 K each; K-blocked: blocks 2s + kh).
  // One register set per half: a half is reloaded with the next step's as
  // soon as its MFMAs are issued, one half-step (32 MFMAs) ahead of its use.
  v4i abuf[2][4];   // [kh][mt]
  v4i breg[2][2];
  auto load_a = [&](int kh, int s) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      abuf[kh][mt] = *reinterpret_cast<const v4i*>(
          arow[mt] + (KBLK_A ? (size_t)(2 * s + kh) * g.lda : (size_t)s * TKR + TK * kh));
  };
  auto load_b = [&](int s) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        breg[c][h] = *reinterpret_cast<const v4i*>(brow[c] + (size_t)s * TKR + 32 * h);
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<v4i*>(&bs[buf][((tid >> 2) + 64 * c) * BR_LD + 8 * (tid & 3) + 32 * h]) =
            breg[c][h];
  };
  auto compute = [&](int kh, int buf) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const v8bf b = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(
                                                  &bs[buf][(16 * nt + l16) * BR_LD + TK * kh + 8 * q4]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt][nt] = mfma16(__builtin_bit_cast(v8bf, abuf[kh][mt]), b, acc[mt][nt]);
    }
  };

  if (nks > 0) {
    load_b(0);
    load_a(0, 0);
    load_a(1, 0);
    store_b(0);
    __syncthreads();
    // step s from LDS buffer s & 1: prefetch B of s+1; per K half, its
    // MFMAs, then the half's A of s+1; stage B of s+1 into the other buffer
    auto step = [&](const int j, const int s) {
      const int sn = min(s + 1, nks - 1);
      load_b(sn);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, j);
      __builtin_amdgcn_sched_barrier(0);
      load_a(0, sn);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, j);
      __builtin_amdgcn_sched_barrier(0);
      load_a(1, sn);
      store_b(j ^ 1);
      __syncthreads();
    };
    int s = 0;
    for (; s + 2 <= nks; s += 2) {
      step(0, s);
      step(1, s + 1);
    }
    if (s < nks) step(0, s);
  }

  // ---------------------------------------------------------- epilogues
  const int ntt = (wi.mcount + 15) >> 4;
  if constexpr (MODE == TM_FWD_GU) {
    // lane: g (acc[h]) and u (acc[h + 2]) of hidden 128 nc + 32 wave + 16 h + 4 q4 + r,
    // row 16 nt + l16.  1x128 amax of g and of u over the workgroup's 128 hidden
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      float mg = 0.f, mu = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mg = fmaxf(mg, fabsf(acc[h][nt][r]));
          mu = fmaxf(mu, fabsf(acc[h + 2][nt][r]));
        }
      mg = fmaxf(mg, __shfl_xor(mg, 16));
      mg = fmaxf(mg, __shfl_xor(mg, 32));
      mu = fmaxf(mu, __shfl_xor(mu, 16));
      mu = fmaxf(mu, __shfl_xor(mu, 32));
      if (lane < 16) {
        red[((wave * 8 + nt) * 16 + lane) * 2] = mg;
        red[((wave * 8 + nt) * 16 + lane) * 2 + 1] = mu;
      }
    }
    __syncthreads();
    const int I = g.I, nblk = I / QBLK;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int m = 16 * nt + l16;
      if (nt < ntt && m < wi.mcount) {
        float ag = 0.f, au = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ag = fmaxf(ag, red[((w * 8 + nt) * 16 + l16) * 2]);
          au = fmaxf(au, red[((w * 8 + nt) * 16 + l16) * 2 + 1]);
        }
        const float sg = fp8_scale(ag), su = fp8_scale(au);
        const size_t r = (size_t)(wi.row0 + m);
        uint8_t* qrow = g.guq + r * (size_t)(2 * I);
        uint16_t* arow_o = g.abf + r * (size_t)I;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 128 * wi.nc + 32 * wave + 16 * h + 4 * q4;
          const v4f gv = acc[h][nt], uv = acc[h + 2][nt];
          *reinterpret_cast<uint32_t*>(qrow + j) =
              cvt4_e4m3(clamp_fp8(gv[0] / sg), clamp_fp8(gv[1] / sg), clamp_fp8(gv[2] / sg),
                        clamp_fp8(gv[3] / sg));
          *reinterpret_cast<uint32_t*>(qrow + I + j) =
              cvt4_e4m3(clamp_fp8(uv[0] / su), clamp_fp8(uv[1] / su), clamp_fp8(uv[2] / su),
                        clamp_fp8(uv[3] / su));
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = gv[i] / (1.0f + expf(-gv[i])) * uv[i];
          *reinterpret_cast<uint2*>(arow_o + j) =
              make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        }
        if (wave == 0 && q4 == 0) {
          float* srow = g.gus + r * (size_t)(2 * nblk);
          srow[wi.nc] = sg;
          srow[nblk + wi.nc] = su;
        }
      }
    }
  } else if constexpr (MODE == TM_FWD_DOWN || MODE == TM_BWD_GU) {
    // fp32 rows: routed rows (times their routing weight in the forward) to
    // rows[r], shared rows to shared[r - P]
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int m = 16 * nt + l16;
      if (nt < ntt && m < wi.mcount) {
        const int r = wi.row0 + m;
        const bool sh = r >= g.P;
        float wt = 1.f;
        if (MODE == TM_FWD_DOWN && !sh) wt = g.topk_w[min(max(g.row_pair[r], 0), g.P - 1)];
        float* dst = sh ? g.shared_out + (size_t)(r - g.P) * g.ldo : g.rows + (size_t)r * g.ldo;
        dst += 256 * wi.nc + TMW * wave + 4 * q4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          v4f o = acc[mt][nt];
          if (MODE == TM_FWD_DOWN) {
            o[0] = __fmul_rn(o[0], wt); o[1] = __fmul_rn(o[1], wt);
            o[2] = __fmul_rn(o[2], wt); o[3] = __fmul_rn(o[3], wt);
          }
          *reinterpret_cast<float4*>(dst + 16 * mt) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  } else {   // TM_BWD_DOWN
    // lane: da_raw of hidden i = 256 nc + 64 wave + 16 mt + 4 q4 + r, row 16 nt + l16.
    // a~ = silu(g~) u~ from the stored copies; the routing weight's gradient
    // a~ . da_raw is summed over this workgroup's 256 hidden (one partial per
    // (row, chunk)); da = w da_raw; dg, du and a~ leave as bf16.
    const int I = g.I, nblk = I / QBLK;
    float part[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      part[nt] = 0.f;
      const int m = 16 * nt + l16;
      const int r = wi.row0 + min(m, wi.mcount - 1);
      const bool live = nt < ntt && m < wi.mcount;
      const bool sh = r >= g.P;
      const float wt = sh ? 1.f : g.topk_w[min(max(g.row_pair[r], 0), g.P - 1)];
      const uint8_t* qrow = g.guq + (size_t)r * (2 * I);
      const float* srow = g.gus + (size_t)r * (2 * nblk);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int i = 256 * wi.nc + TMW * wave + 16 * mt + 4 * q4;
        const uint32_t gc = *reinterpret_cast<const uint32_t*>(qrow + i);
        const uint32_t uc = *reinterpret_cast<const uint32_t*>(qrow + I + i);
        const float sg = srow[i / QBLK], su = srow[nblk + i / QBLK];
        float dg[4], du[4], av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gt = e4m3_byte(gc, e) * sg;
          const float ut = e4m3_byte(uc, e) * su;
          const float sgm = 1.0f / (1.0f + expf(-gt));
          const float silu = gt * sgm;
          av[e] = silu * ut;
          const float dr = acc[mt][nt][e];
          part[nt] += av[e] * dr;
          const float da = wt * dr;
          dg[e] = da * ut * (sgm * (1.0f + gt * (1.0f - sgm)));
          du[e] = da * silu;
        }
        if (live) {
          uint16_t* drow = g.dgu + (size_t)r * (2 * I);
          *reinterpret_cast<uint2*>(drow + i) =
              make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(drow + I + i) =
              make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
          *reinterpret_cast<uint2*>(g.abf + (size_t)r * I + i) =
              make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
        }
      }
      part[nt] += __shfl_xor(part[nt], 16);
      part[nt] += __shfl_xor(part[nt], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) red[(wave * 8 + nt) * 16 + lane] = part[nt];
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int m = 16 * nt + lane;
        if (nt < ntt && m < wi.mcount) {
          const float s = ((red[(0 * 8 + nt) * 16 + lane] + red[(1 * 8 + nt) * 16 + lane]) +
                           red[(2 * 8 + nt) * 16 + lane]) + red[(3 * 8 + nt) * 16 + lane];
          g.dwp[(size_t)(wi.row0 + m) * g.NC + wi.nc] = s;
        }
      }
    }
  }
}

// ------------------------------------------------- transposes and padding
// Padded column offsets of the groups in the transposed operands: group gi
// takes ceil(len / 32) * 32 columns (zero-filled past its rows).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(int E, int G, int T, int P,
                                                           const int32_t* offsets,
                                                           int32_t* pad_off) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  int total = 0;
  // one thread per group (G <= 1025: the last thread takes two)
  auto len_of = [&](int gi) {
    if (gi >= G) return 0;
    if (gi >= E) return T;
    return min(max(offsets[gi + 1] - offsets[gi], 0), P);
  };
  const int a = len_of(t), b = (t == 1023) ? len_of(1024) : 0;
  const int mine = ((a + 31) & ~31) + ((b + 31) & ~31);
  sums[t] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  total = sums[t] - mine;   // exclusive prefix
  if (t < G) pad_off[t] = total;
  if (t == 1023 && G > 1024) pad_off[1024] = total + ((a + 31) & ~31);
  if (t == 1023) pad_off[G] = sums[1023];
}

// Transposed, group-padded copy of per-row data, K-blocked: padded column q
// of feature c at ((q / 32) * C + c) * 32 + q % 32, so the 32 columns of a
// K step are 64 contiguous bytes per feature and consecutive features follow
// each other (a 16-feature load of one step reads 1 KB contiguous, whole
// cache lines).  Column pad_off[g] + j holds row offsets-of-g + j.  Modes:
//   0: bf16 source rows src[r][C]
//   1: bf16 w_r * dy[token(r)] (routed rows times their routing weight)
//   2: h~ = bf16(e4m3 code * scale) of token(r) from the stored FP8 h
template <int SRC>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const TransposeArgs a) {
  __shared__ uint16_t tile[64][66];
  __shared__ int g_first;
  const int c0 = blockIdx.y * 64;
  const int q0 = blockIdx.x * 64;   // padded column block
  const int tid = threadIdx.x;
  // group of padded column q0 (largest g with pad_off[g] <= q0), searched
  // once per workgroup; the block's 64 columns span few groups
  if (tid == 0) {
    int lo = 0, hi = a.G;   // pad_off[0] = 0 <= q0 < pad_off[G] for q0 inside
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.pad_off[mid] <= q0) lo = mid; else hi = mid;
    }
    g_first = lo;
  }
  __syncthreads();
  // stage: thread reads 16 consecutive features of one padded row
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const int q = q0 + rr;
    // group of padded column q: walk forward from the block's first group
    int gi = g_first;
    while (gi + 1 < a.G && a.pad_off[gi + 1] <= q) ++gi;
    const int j = q - a.pad_off[gi];
    int len, r0;
    if (gi >= a.E) { r0 = a.P; len = a.T; } else {
      r0 = min(max(a.offsets[gi], 0), a.P);
      len = min(max(a.offsets[gi + 1] - r0, 0), a.P - r0);
    }
    const bool valid = q < a.pad_off[a.G] && j < len;
    uint16_t v[16];
    if (!valid) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0;
    } else {
      const int r = r0 + j;
      if constexpr (SRC == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(a.src + (size_t)r * a.C + c0 + cc);
        const uint4 x0 = p[0], x1 = p[1];
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) { v[2 * i] = w[i] & 0xFFFF; v[2 * i + 1] = w[i] >> 16; }
      } else {
        const bool sh = r >= a.P;
        int tok = sh ? r - a.P : a.row_pair[r] / a.k;
        tok = min(max(tok, 0), a.T - 1);
        if constexpr (SRC == 1) {
          const float wt = sh ? 1.f : a.topk_w[min(max(a.row_pair[r], 0), a.P - 1)];
          const uint4* p = reinterpret_cast<const uint4*>(a.src + (size_t)tok * a.C + c0 + cc);
          const uint4 x0 = p[0], x1 = p[1];
          const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            v[2 * i] = (uint16_t)f32_to_bf16_rne(wt * bf16_to_f32(w[i] & 0xFFFF));
            v[2 * i + 1] = (uint16_t)f32_to_bf16_rne(wt * bf16_to_f32(w[i] >> 16));
          }
        } else {
          const uint4 cw = *reinterpret_cast<const uint4*>(a.codes + (size_t)tok * a.C + c0 + cc);
          const float sc = a.scales[(size_t)tok * (a.C / QBLK) + (c0 + cc) / QBLK];
          const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[i] = (uint16_t)f32_to_bf16_rne(e4m3_byte(w[i >> 2], i & 3) * sc);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[rr][cc + i] = v[i];
  }
  __syncthreads();
  // write: thread writes 16 consecutive padded columns of one feature
  {
    const int cr = tid >> 2, qq = (tid & 3) * 16;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (uint32_t)tile[qq + 2 * i][cr] | ((uint32_t)tile[qq + 2 * i + 1][cr] << 16);
    const int q = q0 + qq;   // 16 columns inside one 32-column block
    uint4* dst = reinterpret_cast<uint4*>(a.dst + ((size_t)(q >> 5) * a.C + c0 + cr) * 32 + (q & 31));
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Transpose of bf16 matrices into the K-blocked layout the dgrad products
// read: dst (c, k) = src[k - dst_col0][c] for one [R][C] matrix per
// blockIdx.z, element (c, k) at ((k / 32) * C + c) * 32 + k % 32 (dst_col0:
// the K offset, for stacking gate and up); src_ld in elements.
__global__ __launch_bounds__(256) void transpose_w_kernel(int R, int C, const uint16_t* src,
                                                          size_t src_stride, int src_ld,
                                                          uint16_t* dst, size_t dst_stride,
                                                          int dst_col0) {
  __shared__ uint16_t tile[64][66];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* s = src + (size_t)blockIdx.z * src_stride;
  uint16_t* d = dst + (size_t)blockIdx.z * dst_stride;
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const uint4* p = reinterpret_cast<const uint4*>(s + (size_t)(r0 + rr) * src_ld + c0 + cc);
    const uint4 x0 = p[0], x1 = p[1];
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tile[rr][cc + 2 * i] = w[i] & 0xFFFF;
      tile[rr][cc + 2 * i + 1] = w[i] >> 16;
    }
  }
  __syncthreads();
  {
    const int cr = tid >> 2, qq = (tid & 3) * 16;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (uint32_t)tile[qq + 2 * i][cr] | ((uint32_t)tile[qq + 2 * i + 1][cr] << 16);
    const int k = dst_col0 + r0 + qq;   // 16 K inside one 32-wide block
    uint4* o = reinterpret_cast<uint4*>(d + ((size_t)(k >> 5) * C + c0 + cr) * 32 + (k & 31));
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// ------------------------------------------------------------- routing
// s of the chosen experts, as the top-k kernel forms it from the summed logits
__global__ __launch_bounds__(256) void chosen_scores_kernel(int T, int E, int k, const float* z,
                                                            const int32_t* ids, float* s) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * k) return;
  const int t = i / k;
  const int e = min(max(ids[i], 0), E - 1);
  s[i] = (float)(1.0 / (1.0 + exp(-(double)z[(size_t)t * E + e])));
}

// Router and RMSNorm backward, one workgroup per token:
//   dw_j  = sum of the routed row's partials (fixed chunk order)
//   ds_j  = c (dw_j / S - sum_i dw_i s_i / S^2)   (c dw_j without renormalisation)
//   dz_j  = ds_j s_j (1 - s_j)
//   dh    = dh_experts + sum_j dz_j W_r[id_j]
//   dx    = dout + r gamma dh - x r^3 / d sum(gamma dh x)
//   dgamma partial of the token: dh x r (summed over tokens afterwards)
__global__ __launch_bounds__(256) void router_norm_bwd_kernel(const RouterBwdArgs a) {
  __shared__ float dz_sh[32];
  __shared__ double red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k, d = a.d;
  if (tid == 0) {
    float dw[32], s[32];
    double S = 0.0, sds = 0.0;
    for (int j = 0; j < k; ++j) {
      const int p = t * k + j;
      const int r = min(max(a.pair_row[p], 0), a.P - 1);
      float acc = 0.f;
      for (int c = 0; c < a.nchunk; ++c) acc += a.dwp[(size_t)r * a.nchunk + c];
      dw[j] = acc;
      s[j] = a.s[p];
      S += (double)s[j];
      sds += (double)dw[j] * (double)s[j];
    }
    for (int j = 0; j < k; ++j) {
      const double ds = a.renorm ? (double)a.scaling * ((double)dw[j] / S - sds / (S * S))
                                 : (double)a.scaling * (double)dw[j];
      const float dz = (float)(ds * (double)s[j] * (1.0 - (double)s[j]));
      dz_sh[j] = dz;
      a.dz[t * k + j] = dz;
      if (a.dw_out) a.dw_out[t * k + j] = dw[j];
    }
  }
  __syncthreads();
  // dh (fp32) + router rows, then the RMSNorm backward
  const uint16_t* xr = a.x + (size_t)t * d;
  double ss = 0.0, dot = 0.0;
  for (int c = tid; c < d; c += 256) {
    const float xv = bf16_to_f32(xr[c]);
    ss += (double)xv * (double)xv;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double ms = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  const double rr = 1.0 / sqrt(ms / d + (double)a.eps);
  for (int c = tid; c < d; c += 256) {
    double dh = (double)a.dh[(size_t)t * d + c];
    for (int j = 0; j < k; ++j) {
      const int e = min(max(a.ids[t * k + j], 0), a.E - 1);
      dh += (double)dz_sh[j] * (double)bf16_to_f32(a.w_router[(size_t)e * d + c]);
    }
    const double xv = bf16_to_f32(xr[c]);
    dot += (double)bf16_to_f32(a.norm_w[c]) * dh * xv;
    a.dh_total[(size_t)t * d + c] = (float)dh;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
  if (lane == 0) red[wave] = dot;
  __syncthreads();
  const double sdot = (red[0] + red[1]) + (red[2] + red[3]);
  const double coef = rr * rr * rr / d * sdot;
  for (int c = tid; c < d; c += 256) {
    const double dh = (double)a.dh_total[(size_t)t * d + c];
    const double xv = bf16_to_f32(xr[c]);
    const double gam = bf16_to_f32(a.norm_w[c]);
    const double dout = bf16_to_f32(a.dout[(size_t)t * d + c]);
    a.dx[(size_t)t * d + c] = (float)(dout + rr * gam * dh - xv * coef);
    a.dh_total[(size_t)t * d + c] = (float)(dh * xv * rr);   // this token's dgamma term
  }
}

// Column sums over tokens in a fixed order, in fp64: partial sums over
// chunks of COL_CHUNK tokens (one thread per column and chunk), then the
// chunks in ascending order.
constexpr int COL_CHUNK = 128;
__global__ __launch_bounds__(256) void col_partial_kernel(int T, int d, const float* in,
                                                          double* part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const int t0 = blockIdx.y * COL_CHUNK, t1 = min(t0 + COL_CHUNK, T);
  double s = 0.0;
  for (int t = t0; t < t1; ++t) s += (double)in[(size_t)t * d + c];
  part[(size_t)blockIdx.y * d + c] = s;
}

__global__ __launch_bounds__(256) void col_sum_kernel(int nchunk, int d, const double* part,
                                                      float* out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double s = 0.0;
  for (int k = 0; k < nchunk; ++k) s += part[(size_t)k * d + c];
  out[c] = (float)s;
}

// Router weight gradient: dW_r[e][c] = sum over the rows of expert e (in
// permuted order) of dz of that (token, slot) times h~[token][c]
__global__ __launch_bounds__(256) void router_wgrad_kernel(int E, int d, int k, int P,
                                                           const int32_t* offsets,
                                                           const int32_t* row_pair,
                                                           const float* dz, const uint8_t* hq,
                                                           const float* hs, float* dwr) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 1024 + 4 * threadIdx.x;
  if (c >= d) return;
  const int r0 = min(max(offsets[e], 0), P), r1 = min(max(offsets[e + 1], r0), P);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < r1; ++r) {
    const int p = min(max(row_pair[r], 0), P - 1);
    const int t = p / k;
    const float g = dz[p];
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(hq + (size_t)t * d + c);
    const float sc = hs[(size_t)t * (d / QBLK) + c / QBLK];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] += g * bf16_to_f32(f32_to_bf16_rne(e4m3_byte(cw, i) * sc));
  }
  *reinterpret_cast<float4*>(dwr + (size_t)e * d + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// Weight gradients C[out][in] = sum over a group's rows of X^T Y, in
// WGM x 128 tiles (4 waves of WGM / 4 M rows, 8 16-row N tiles).  A tile's K is a
// group's rows, a few steps of 32 at the routed experts' sizes, so a one-step
// prefetch would leave every step waiting a full memory round trip: the A
// rows and the staged B rows are loaded PF steps ahead into a register ring
// of PF + 1 sets.  The B rows go through LDS (double-buffered) as in
// train_gemm_kernel; the same LDS then turns the results around so that 32
// lanes store one row's 128 columns (512 contiguous bytes).
constexpr int OT_LD = TN + 4;          // fp32 stride of a turned-around row
constexpr int WG_LDS_BYTES = 4 * 16 * OT_LD * 4;
static_assert(WG_LDS_BYTES >= 2 * TN * B_LD * 2, "LDS turnaround must hold the B stages");

template <int PF, int WGM, int MINW>
__global__ __launch_bounds__(256, MINW) void train_wgrad_kernel(const TrainGemmArgs g) {
  constexpr int WG_MW = WGM / 4;       // M rows per wave
  constexpr int WG_MT = WG_MW / 16;    // 16-row M tiles per wave
  constexpr int NR = PF + 1;           // register ring sets
  constexpr int UN = 2 * NR;           // unroll: LDS buffer and ring slot compile-time
  __shared__ __attribute__((aligned(16))) uint8_t lds[WG_LDS_BYTES];
  uint16_t* bs = reinterpret_cast<uint16_t*>(lds);   // [2][TN * B_LD] during the K loop
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;

  const TileWork wi = decode_wgrad(g);
  if (!wi.valid) return;
  const int grp = wi.grp;
  const int k0 = g.pad_off[grp], k1 = g.pad_off[grp + 1];
  const size_t kbase = (size_t)k0;
  const int nks = (k1 - k0) / TK;

  // K-blocked operands: step s of row r at (kbase / 32 + s) * ld + 32 r
  const uint16_t* arow[WG_MT];
#pragma unroll
  for (int mt = 0; mt < WG_MT; ++mt) {
    const size_t row = (size_t)(WGM * wi.mi + WG_MW * wave + 16 * mt + l16);
    arow[mt] = g.A + (kbase / TK) * (size_t)g.lda + row * TK + 8 * q4;
  }
  const uint16_t* brow[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int tr = (tid >> 2) + 64 * c;
    brow[c] = g.B + (kbase / TK) * (size_t)g.ldb + (size_t)(TN * wi.ni + tr) * TK + 8 * (tid & 3);
  }

  v4f acc[WG_MT][8];
#pragma unroll
  for (int mt = 0; mt < WG_MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i ar[NR][WG_MT];
  v4i br[NR][2];
  // loads of step s (clamped to the last step: past it they repeat loads
  // that are never used)
  auto load = [&](int slot_a, int s) {
    const int sc = min(s, nks - 1);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      br[slot_a][c] = *reinterpret_cast<const v4i*>(brow[c] + (size_t)sc * g.ldb);
#pragma unroll
    for (int mt = 0; mt < WG_MT; ++mt)
      ar[slot_a][mt] = *reinterpret_cast<const v4i*>(arow[mt] + (size_t)sc * g.lda);
  };
  auto store_b = [&](int buf, int slot) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      *reinterpret_cast<v4i*>(&bs[buf * TN * B_LD + ((tid >> 2) + 64 * c) * B_LD + 8 * (tid & 3)]) =
          br[slot][c];
  };
  auto compute = [&](int slot, int buf) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const v8bf b = __builtin_bit_cast(
          v8bf, *reinterpret_cast<const v4i*>(&bs[buf * TN * B_LD + (16 * nt + l16) * B_LD + 8 * q4]));
#pragma unroll
      for (int mt = 0; mt < WG_MT; ++mt)
        acc[mt][nt] = mfma16(__builtin_bit_cast(v8bf, ar[slot][mt]), b, acc[mt][nt]);
    }
  };

  if (nks > 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) load(j, j);   // steps 0 .. PF
    store_b(0, 0);
    __syncthreads();
    // step s (ring slot s % NR, LDS buffer s % 2): compute, stage B of s + 1
    // into the other buffer, load step s + NR into the freed slot
    for (int s0 = 0; s0 < nks; s0 += UN) {
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        const int s = s0 + j;
        if (s < nks) {
          compute(j % NR, j & 1);
          store_b((j + 1) & 1, (j + 1) % NR);
          load(j % NR, s + NR);
          __syncthreads();
        }
      }
    }
  }
  // after the last step's barrier (or with no K steps, LDS untouched) the
  // LDS turns C[m][n] around -> out[grp][m][n] (fp32, nn.Linear layout),
  // non-temporal (the gradient is not read again here)
  float* out = g.out + (size_t)grp * g.out_stride + (size_t)TN * wi.ni;
  float* tw = reinterpret_cast<float*>(lds) + wave * 16 * OT_LD;
#pragma unroll
  for (int mt = 0; mt < WG_MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tw[(4 * q4 + r) * OT_LD + 16 * nt + l16] = acc[mt][nt][r];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 2 * i + (lane >> 5), col = 4 * (lane & 31);
      const v4f v = *reinterpret_cast<const v4f*>(&tw[row * OT_LD + col]);
      const size_t m = (size_t)(WGM * wi.mi + WG_MW * wave + 16 * mt + row);
      __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(out + m * g.ldo + col));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// the ring depth used: loads one step ahead (two and three steps ahead
// measured 3% and 7% slower at the K2 prefill batch, bitwise the same)
constexpr int WGRAD_PF = 1;
// waves per SIMD the register budget is sized for: two workgroups per CU.
// 128-row tiles at four per CU (116 registers) were no faster and slowed the
// input-gradient products that run beside them on the other stream.
constexpr int WGRAD_MINW = WGRAD_M == 256 ? 2 : 4;

}  // namespace

hipError_t launch_train_gemm(int mode, const TrainGemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (mode) {
    case TM_FWD_GU: train_gemm_kernel<TM_FWD_GU><<<grid, 256, 0, s>>>(a); break;
    case TM_FWD_DOWN: train_gemm_kernel<TM_FWD_DOWN><<<grid, 256, 0, s>>>(a); break;
    case TM_BWD_DOWN: train_gemm_kernel<TM_BWD_DOWN><<<grid, 256, 0, s>>>(a); break;
    case TM_BWD_GU: train_gemm_kernel<TM_BWD_GU><<<grid, 256, 0, s>>>(a); break;
    case TM_WGRAD:
      train_wgrad_kernel<WGRAD_PF, WGRAD_M, WGRAD_MINW><<<grid, 256, 0, s>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pad_offsets(int E, int G, int T, int P, const int32_t* offsets,
                              int32_t* pad_off, hipStream_t s) {
  pad_offsets_kernel<<<1, 1024, 0, s>>>(E, G, T, P, offsets, pad_off);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(int src_mode, const TransposeArgs& a, int padded_cols,
                                hipStream_t s) {
  const dim3 grid((unsigned)((padded_cols + 63) / 64), (unsigned)(a.C / 64));
  switch (src_mode) {
    case 0: transpose_pad_kernel<0><<<grid, 256, 0, s>>>(a); break;
    case 1: transpose_pad_kernel<1><<<grid, 256, 0, s>>>(a); break;
    case 2: transpose_pad_kernel<2><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_transpose_w(int n, int R, int C, const uint16_t* src, size_t src_stride,
                              int src_ld, uint16_t* dst, size_t dst_stride, int dst_col0,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  transpose_w_kernel<<<dim3(R / 64, C / 64, n), 256, 0, s>>>(R, C, src, src_stride, src_ld, dst,
                                                             dst_stride, dst_col0);
  return hipGetLastError();
}

hipError_t launch_chosen_scores(int T, int E, int k, const float* z, const int32_t* ids,
                                float* sc, hipStream_t s) {
  const int n = T * k;
  if (n <= 0) return hipSuccess;
  chosen_scores_kernel<<<(n + 255) / 256, 256, 0, s>>>(T, E, k, z, ids, sc);
  return hipGetLastError();
}

hipError_t launch_router_norm_bwd(const RouterBwdArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  router_norm_bwd_kernel<<<a.T, 256, 0, s>>>(a);
  return hipGetLastError();
}

size_t col_sum_scratch_bytes(int T, int d) {
  return (size_t)((T + COL_CHUNK - 1) / COL_CHUNK) * d * sizeof(double);
}

hipError_t launch_col_sum(int T, int d, const float* in, double* scratch, float* out,
                          hipStream_t s) {
  const int nchunk = (T + COL_CHUNK - 1) / COL_CHUNK;
  col_partial_kernel<<<dim3((d + 255) / 256, nchunk), 256, 0, s>>>(T, d, in, scratch);
  col_sum_kernel<<<(d + 255) / 256, 256, 0, s>>>(nchunk, d, scratch, out);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(int E, int d, int k, int P, const int32_t* offsets,
                               const int32_t* row_pair, const float* dz, const uint8_t* hq,
                               const float* hs, float* dwr, hipStream_t s) {
  router_wgrad_kernel<<<dim3(E, (d + 1023) / 1024), 256, 0, s>>>(E, d, k, P, offsets, row_pair,
                                                                 dz, hq, hs, dwr);
  return hipGetLastError();
}

}  // namespace k2
