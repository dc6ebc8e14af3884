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
// rows are gathered into LDS in fragment order (double-buffered).  MFMA:
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
#include "k2_common.h"
#include "k2_launch.h"

namespace k2 {

namespace {

__device__ __forceinline__ v8i join8(v4i a, v4i b) {
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // atype = btype = 0 (e4m3), E8M0 scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

template <bool GATEUP, int TT>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(const GemmArgs g) {
  constexpr int BM = 16 * TT;
  constexpr int CPT = (TT * 128 + 255) / 256;   // 16-byte staging chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][TT * 2048];
  __shared__ float lds_red[GATEUP ? 4 * TT * 16 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------------------------------------------------------- work item
  const int Wtot = g.mt_start[g.G] * g.NC;
  const int Wp = (Wtot + 7) & ~7;
  const int b = blockIdx.x;
  if (b >= Wp) return;
  const int L = (b & 7) * (Wp >> 3) + (b >> 3);
  if (L >= Wtot) return;
  const int q = L / g.NC;
  int lo = 0, hi = g.G;                    // mt_start[lo] <= q < mt_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mt_start[mid] <= q) lo = mid; else hi = mid;
  }
  const int grp = lo;
  const bool shared_grp = grp >= g.E;
  int row0_g, m_g;
  if (shared_grp) {
    row0_g = g.P;
    m_g = g.T;
  } else {
    row0_g = min(max(g.offsets[grp], 0), g.P);
    m_g = min(max(g.offsets[grp + 1] - row0_g, 0), g.P - row0_g);
  }
  const int mtiles = (m_g + BM - 1) / BM;
  const int rr = L - g.mt_start[grp] * g.NC;
  const int nc = rr / mtiles, mt = rr - nc * mtiles;
  const int row0 = row0_g + mt * BM;
  const int mcount = min(BM, m_g - mt * BM);
  const int ntt = (mcount + 15) >> 4;

  // activation row of the m-th row of this tile (padding rows repeat the last)
  auto act_row = [&](int m) -> int {
    const int mm = min(m, mcount - 1);
    if constexpr (GATEUP) {
      if (shared_grp) return row0 + mm - g.P;
      const int tok = g.row_pair[row0 + mm] / g.k;
      return min(max(tok, 0), g.T - 1);
    } else {
      return row0 + mm;
    }
  };

  // staging of the activation tile into LDS, fragment order:
  // [tt][half p][lane][16 B], lane = token%16 + 16 * (32-byte group)
  uint32_t boff[CPT];
  int bdst[CPT];
  bool bon[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    bon[i] = c < TT * 128;
    const int m = c >> 3, piece = c & 7;
    boff[i] = bon[i] ? (uint32_t)act_row(m) * (uint32_t)g.act_ld + piece * 16 : 0u;
    bdst[i] = (m >> 4) * 2048 + (piece & 1) * 1024 + ((m & 15) + 16 * (piece >> 1)) * 16;
  }
  uint32_t saoff[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) saoff[tt] = (uint32_t)act_row(tt * 16 + (lane & 15)) * g.nkb;

  const uint8_t* wp = g.wpk + (size_t)grp * g.expert_stride +
                      (size_t)(nc * 4 + wave) * (size_t)g.nkb * 8192 + lane * 16;
  const float* swp = GATEUP
      ? g.wscale + (size_t)grp * g.wscale_stride + (size_t)nc * g.nkb * 2
      : g.wscale + (size_t)grp * g.wscale_stride + (size_t)(nc * 2 + (wave >> 1)) * g.nkb;

  v4f acc[4][TT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i wA[4], wB[4];
  v4i breg[CPT];
  float saA[TT], saB[TT];
  float swA[2], swB[2];

  auto load_w = [&](v8i (&w)[4], int kb) {
    const uint8_t* p = wp + (size_t)kb * 8192;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const v4i lo4 = *reinterpret_cast<const v4i*>(p + rt * 2048);
      const v4i hi4 = *reinterpret_cast<const v4i*>(p + rt * 2048 + 1024);
      w[rt] = join8(lo4, hi4);
    }
  };
  auto load_b = [&](int kb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (bon[i]) breg[i] = *reinterpret_cast<const v4i*>(g.act + boff[i] + kb * 128);
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (bon[i]) *reinterpret_cast<v4i*>(&lds_b[buf][bdst[i]]) = breg[i];
  };
  auto load_s = [&](float (&sa)[TT], float (&sw)[2], int kb) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) sa[tt] = g.act_s[saoff[tt] + kb];
    if constexpr (GATEUP) {
      sw[0] = swp[2 * kb];
      sw[1] = swp[2 * kb + 1];
    } else {
      sw[0] = swp[kb];
      sw[1] = sw[0];
    }
  };
  auto compute = [&](const v8i (&w)[4], int buf, const float (&sa)[TT], const float (&sw)[2]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < ntt) {
        const uint8_t* bp = &lds_b[buf][tt * 2048 + lane * 16];
        const v8i bf = join8(*reinterpret_cast<const v4i*>(bp),
                             *reinterpret_cast<const v4i*>(bp + 1024));
        const float s0 = sa[tt] * sw[0];
        const float s1 = sa[tt] * sw[1];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v4f f = mfma_fp8(w[rt], bf);
          const float sc = rt < 2 ? s0 : s1;
          acc[rt][tt] += f * sc;
        }
      }
    }
  };

  // ---------------------------------------------------------------- K loop
  const int nkb = g.nkb;
  load_w(wA, 0);
  load_b(0);
  load_s(saA, swA, 0);
  store_b(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    const bool has_next = kb + 1 < nkb;  // block kb+1 exists
    if (has_next) {
      load_w(wB, kb + 1);
      load_b(kb + 1);
      load_s(saB, swB, kb + 1);
    }
    compute(wA, 0, saA, swA);
    if (has_next) store_b(1);
    __syncthreads();
    if (!has_next) break;
    const bool more = kb + 2 < nkb;
    if (more) {
      load_w(wA, kb + 2);
      load_b(kb + 2);
      load_s(saA, swA, kb + 2);
    }
    compute(wB, 1, saB, swB);
    if (more) store_b(0);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
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
          float wt = 1.f;
          const bool mul = g.weighted && !shared_grp;
          if (mul) wt = g.topk_w[min(max(g.row_pair[row], 0), g.P - 1)];
          float* dst = shared_grp ? g.shared_out + (size_t)(row - g.P) * g.d
                                  : g.rows + (size_t)row * g.d;
          dst += nc * 256 + 64 * wave + 4 * (lane >> 4);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            v4f o = acc[rt][tt];
            if (mul) o = o * wt;
            *reinterpret_cast<float4*>(dst + 16 * rt) = make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  }
}

template <bool GATEUP>
hipError_t launch_tt(int tt, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tt) {
    case 1: gemm_fp8_kernel<GATEUP, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: gemm_fp8_kernel<GATEUP, 2><<<grid, 256, 0, s>>>(a); break;
    case 4: gemm_fp8_kernel<GATEUP, 4><<<grid, 256, 0, s>>>(a); break;
    case 8: gemm_fp8_kernel<GATEUP, 8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(bool gateup, int tt, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return gateup ? launch_tt<true>(tt, a, grid, s) : launch_tt<false>(tt, a, grid, s);
}

}  // namespace k2
