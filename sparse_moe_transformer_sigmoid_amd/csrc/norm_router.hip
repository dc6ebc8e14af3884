// RMSNorm + 1x128 FP8 activation quantisation, the bf16 router GEMM and the
// sigmoid / correction-bias top-k selection of the K2 MoE layer.
//
// RMSNorm ("Kimi-K2-Base", Normalization and stability: RMSNorm, pre-norm,
// eps 1e-6): ms = mean(x^2) rounded to fp32 (formed in fp64, so the rounding
// does not depend on the reduction order), r = 1/sqrt(ms + eps) with IEEE
// fp32 ops, h = bf16((x * r) * gamma).
// Quantisation ("Kimi K2 · Architecture", config.json quantization_config,
// activation_scheme dynamic; "Kimi-K2-Base", Training precision, 1x128 tiles
// with fp32 scales): per token and 128 columns, s = amax/448,
// q = e4m3(clamp(h/s, +-448)) with IEEE division.
// Router ("Kimi-K2-Base", Mixture of experts): z = h . W_r^T (bf16 inputs,
// fp32 accumulate), s = sigmoid(z), the correction bias is added for the
// choice only, top-k with one group, weights = s / sum(s) * scaling.
#include "k2_common.h"
#include "k2_launch.h"

namespace k2 {

namespace {

constexpr int NQ_THREADS = 256;
constexpr int NQ_MAXIT = 8;  // d <= 8 * 256 * 8 = 16384

template <bool FP8>
__global__ __launch_bounds__(NQ_THREADS) void norm_quant_kernel(int d, float eps,
                                                                const void* __restrict__ x,
                                                                const void* __restrict__ gamma,
                                                                uint16_t* __restrict__ hbuf,
                                                                void* __restrict__ xq,
                                                                float* __restrict__ xs) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = d >> 3;  // chunks of 8 elements
  float v[NQ_MAXIT][8];
  double ss = 0.0;
#pragma unroll
  for (int it = 0; it < NQ_MAXIT; ++it) {
    const int c = tid + NQ_THREADS * it;
    if (c < nch) {
      if constexpr (FP8) {
        const uint4 p = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(x) + (size_t)t * d)[c];
        const uint32_t w4[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[it][2 * j] = bf16_to_f32(w4[j] & 0xFFFFu);
          v[it][2 * j + 1] = bf16_to_f32(w4[j] >> 16);
        }
      } else {
        const float4* xp = reinterpret_cast<const float4*>(
            static_cast<const float*>(x) + (size_t)t * d + (size_t)c * 8);
        const float4 a = xp[0], b = xp[1];
        v[it][0] = a.x; v[it][1] = a.y; v[it][2] = a.z; v[it][3] = a.w;
        v[it][4] = b.x; v[it][5] = b.y; v[it][6] = b.z; v[it][7] = b.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += (double)v[it][j] * (double)v[it][j];
    }
  }
  __shared__ double red[NQ_THREADS / WAVE];
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < NQ_THREADS / WAVE; ++w) tot += red[w];
  const float ms = (float)(tot / (double)d);
  const float r = 1.0f / sqrtf(ms + eps);

#pragma unroll
  for (int it = 0; it < NQ_MAXIT; ++it) {
    const int c = tid + NQ_THREADS * it;
    if (c < nch) {
      float h[8];
      if constexpr (FP8) {
        const uint4 gp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(gamma))[c];
        const uint32_t g4[4] = {gp.x, gp.y, gp.z, gp.w};
        uint32_t hb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float g0 = bf16_to_f32(g4[j] & 0xFFFFu), g1 = bf16_to_f32(g4[j] >> 16);
          const uint32_t b0 = f32_to_bf16_rne((v[it][2 * j] * r) * g0);
          const uint32_t b1 = f32_to_bf16_rne((v[it][2 * j + 1] * r) * g1);
          h[2 * j] = bf16_to_f32(b0);
          h[2 * j + 1] = bf16_to_f32(b1);
          hb[j] = b0 | (b1 << 16);
        }
        reinterpret_cast<uint4*>(hbuf + (size_t)t * d)[c] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
        // 16 consecutive lanes hold one 128-column block
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[j]));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        const float sc = fp8_scale(amax);
        const uint32_t q0 = cvt4_e4m3(clamp_fp8(h[0] / sc), clamp_fp8(h[1] / sc),
                                      clamp_fp8(h[2] / sc), clamp_fp8(h[3] / sc));
        const uint32_t q1 = cvt4_e4m3(clamp_fp8(h[4] / sc), clamp_fp8(h[5] / sc),
                                      clamp_fp8(h[6] / sc), clamp_fp8(h[7] / sc));
        reinterpret_cast<uint2*>(static_cast<uint8_t*>(xq) + (size_t)t * d)[c] =
            make_uint2(q0, q1);
        if ((c & 15) == 0) xs[(size_t)t * (d / QBLK) + (c >> 4)] = sc;
      } else {
        const float* gp = static_cast<const float*>(gamma) + (size_t)c * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (v[it][j] * r) * gp[j];
        float4* op = reinterpret_cast<float4*>(static_cast<float*>(xq) + (size_t)t * d +
                                               (size_t)c * 8);
        op[0] = make_float4(h[0], h[1], h[2], h[3]);
        op[1] = make_float4(h[4], h[5], h[6], h[7]);
      }
    }
  }
}

// z partial sums: zpart[ks][t][e] over columns [ks*kchunk, (ks+1)*kchunk).
// Workgroup: 64 tokens x RG_E experts.  The tokens' h columns are staged
// through LDS 128 columns at a time (double-buffered, in MFMA fragment order)
// and shared by the 4 waves; wave w streams the router rows of experts
// e0 + 48w .. e0 + 48w + 47 straight from global memory (the 5.5 MB router
// matrix stays in L2) and keeps 3 x 4 tiles of 16 experts x 16 tokens.
// MFMA v_mfma_f32_16x16x32_bf16: A = 16 router rows, B = 16 tokens, lane l
// holds k = 8 (l / 16) .. + 7 of row / token l % 16.
constexpr int RG_E = 192;
constexpr int RG_KC = 128;

__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(int T, int d, int E, int kchunk,
                                                              const uint16_t* __restrict__ h,
                                                              const uint16_t* __restrict__ wr,
                                                              float* __restrict__ zpart) {
  // [buffer][token tile tt][k32 step s][lane][16 B]
  __shared__ __attribute__((aligned(16))) uint8_t hs[2][4 * 4 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * RG_E + 48 * wave;
  const int ks = blockIdx.z;
  const int kbeg = ks * kchunk;
  const int nch = kchunk / RG_KC;

  // staging: thread tid moves LDS chunk q = tid + 256 i (i = token tile):
  // token 16 i + lane % 16, columns 32 s + 8 (lane / 16) .. + 7 with s = tid / 64
  const int s_st = tid >> 6;
  const uint16_t* hsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = min(t0 + 16 * i + (lane & 15), T - 1);
    hsrc[i] = h + (size_t)tok * d + kbeg + 32 * s_st + 8 * (lane >> 4);
  }
  const uint16_t* wsrc[3];
  bool fon[3];
#pragma unroll
  for (int f = 0; f < 3; ++f) {
    fon[f] = e0 + 16 * f < E;
    const int e = min(e0 + 16 * f + (lane & 15), E - 1);
    wsrc[f] = wr + (size_t)e * d + kbeg + 8 * (lane >> 4);
  }
  v4f acc[3][4];
#pragma unroll
  for (int f = 0; f < 3; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i stage[4];
  auto load_h = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[i] = *reinterpret_cast<const v4i*>(hsrc[i] + c * RG_KC);
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<v4i*>(&hs[buf][(tid + 256 * i) * 16]) = stage[i];
  };
  // router-row fragments of one 128-column chunk, loaded one chunk ahead
  v8bf wa[2][3][4];
  auto load_w = [&](v8bf (&a)[3][4], int c) {
#pragma unroll
    for (int f = 0; f < 3; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[f][s] = *reinterpret_cast<const v8bf*>(wsrc[f] + c * RG_KC + 32 * s);
  };
  auto chunk = [&](const v8bf (&a)[3][4], v8bf (&an)[3][4], int c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) {
      load_h(c + 1);
      load_w(an, c + 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v8bf b = *reinterpret_cast<const v8bf*>(&hs[buf][((i * 4 + s) * 64 + lane) * 16]);
#pragma unroll
        for (int f = 0; f < 3; ++f)
          acc[f][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f][s], b, acc[f][i], 0, 0, 0);
      }
    }
    if (more) store_h(buf ^ 1);
    __syncthreads();
  };
  load_h(0);
  load_w(wa[0], 0);
  store_h(0);
  __syncthreads();
  int c = 0;
  for (; c + 2 <= nch; c += 2) {
    chunk(wa[0], wa[1], c);
    chunk(wa[1], wa[0], c + 1);
  }
  if (c < nch) chunk(wa[0], wa[1], c);
  // lane holds rows (experts) 4 (lane / 16) + r of each tile, column (token) lane % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + 16 * i + (lane & 15);
    if (tt >= T) continue;
#pragma unroll
    for (int f = 0; f < 3; ++f) {
      if (!fon[f]) continue;
      const int e = e0 + 16 * f + 4 * (lane >> 4);
      float4* zp = reinterpret_cast<float4*>(zpart + ((size_t)ks * T + tt) * E + e);
      *zp = make_float4(acc[f][i][0], acc[f][i][1], acc[f][i][2], acc[f][i][3]);
    }
  }
}

__global__ __launch_bounds__(256) void router_gemm_f32_kernel(int T, int d, int E,
                                                             const float* __restrict__ h,
                                                             const float* __restrict__ wr,
                                                             float* __restrict__ z) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * E) return;
  const int t = i / E, e = i - t * E;
  const float* hp = h + (size_t)t * d;
  const float* wp = wr + (size_t)e * d;
  float acc = 0.f;
  for (int j = 0; j < d; ++j) acc = fmaf(hp[j], wp[j], acc);
  z[i] = acc;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

constexpr int TK_WAVES = 4;

// One DPP row shift of a 64-bit value: lane i of each 16-lane row gets lane
// i - S of the same row, and 0 where that lane is outside the row.
template <int S>
__device__ __forceinline__ uint64_t row_shr_u64(uint64_t v) {
  constexpr int ctrl = 0x110 + S;   // DPP row_shr:S
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, ctrl, 0xF, 0xF, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), ctrl, 0xF, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Wave maximum of non-negative 64-bit keys, the same value in every lane.
// Shifts by 1, 2, 4 and 8 within each row leave lane 16r + 15 with the
// maximum of row r; the four row maxima are then read as scalars.  Register
// moves only: no LDS round trips as with a shuffle per step.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  uint64_t o;
  o = row_shr_u64<1>(v); v = o > v ? o : v;
  o = row_shr_u64<2>(v); v = o > v ? o : v;
  o = row_shr_u64<4>(v); v = o > v ? o : v;
  o = row_shr_u64<8>(v); v = o > v ? o : v;
  uint64_t m = lane_u64(v, 15);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    o = lane_u64(v, 16 * r + 15);
    m = o > m ? o : m;
  }
  return m;
}

// One wavefront per token.  Key = (ordered biased score << 32) | ~expert, so
// the wave maximum is the highest score and, on equal scores, the lower id.
template <int MAXJ, int MAXK>
__global__ __launch_bounds__(TK_WAVES * 64) void topk_kernel(int T, int E, int k, int ksplit,
                                                            const float* __restrict__ zpart,
                                                            const float* __restrict__ bias,
                                                            float scaling, int renorm,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ wout,
                                                            float* __restrict__ gap) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t_raw = blockIdx.x * TK_WAVES + wave;
  const int t = min(t_raw, T - 1);
  __shared__ float s_sh[TK_WAVES][MAXJ * 64];
  uint64_t key[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0;
    if (e < E) {
      float z = 0.f;
      for (int ks = 0; ks < ksplit; ++ks) z += zpart[((size_t)ks * T + t) * E + e];
      const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
      const float sb = s + bias[e];
      s_sh[wave][e] = s;
      key[j] = ((uint64_t)ordered_bits(sb) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  __syncthreads();
  int sel[MAXK];
  float sel_sb[MAXK + 1];
  const int rounds = min(k + 1, E);
#pragma unroll
  for (int r = 0; r < MAXK + 1; ++r) {
    if (r < rounds) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) best = key[j] > best ? key[j] : best;
      best = wave_max_key(best);
#pragma unroll
      for (int j = 0; j < MAXJ; ++j)
        if (key[j] == best) key[j] = 0;
      if (r < MAXK) sel[r] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
      sel_sb[r] = unordered_bits((uint32_t)(best >> 32));
    }
  }
  // ascending ids: lane r < k places its expert at its rank among the chosen
  int my_e = 0;
  double my_s = 0.0;
#pragma unroll
  for (int r = 0; r < MAXK; ++r)
    if (r < k && lane == r) my_e = sel[r];
  int rank = 0;
#pragma unroll
  for (int r = 0; r < MAXK; ++r)
    if (r < k && sel[r] < my_e) ++rank;
  float s_me = 0.f;
  if (lane < k) {
    s_me = s_sh[wave][my_e];
    my_s = (double)s_me;
  }
  // sum of the k chosen scores (lanes 0..k-1) in fp64: exact, so in any order,
  // while the scores lie within 2^29 of one another
  double ssum = 0.0;
#pragma unroll
  for (int r = 0; r < MAXK; ++r)
    if (r < k) ssum += __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(my_s), r),
                                        __builtin_amdgcn_readlane(__double2loint(my_s), r));
  const float denom = (float)ssum;
  if (t_raw < T) {
    if (lane < k) {
      const float wv = renorm ? (s_me / denom) * scaling : s_me * scaling;
      ids[(size_t)t * k + rank] = my_e;
      wout[(size_t)t * k + rank] = wv;
    }
    if (gap != nullptr && lane == 0) {
      float g = __builtin_inff();
#pragma unroll
      for (int r = 0; r < MAXK; ++r)
        if (r == k - 1 && k < E) g = sel_sb[r] - sel_sb[r + 1];
      gap[t] = g;
    }
  }
}

// Split-K router partials -> logits, in place in slice 0: one thread per
// (token, expert), partials added in ascending split order.
__global__ __launch_bounds__(256) void zsum_kernel(long n, int ksplit, float* __restrict__ zpart) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float z = 0.f;
  // loads issued 16 at a time; the additions stay in ascending split order
#pragma unroll 16
  for (int ks = 0; ks < ksplit; ++ks) z += zpart[(size_t)ks * n + i];
  zpart[i] = z;
}

__global__ void dense_route_kernel(int T, float scaling, int32_t* ids, float* w, float* gap) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  ids[t] = 0;
  w[t] = scaling;
  if (gap) gap[t] = __builtin_inff();
}

}  // namespace

hipError_t launch_norm_quant(bool fp8, int T, int d, float eps, const void* x, const void* gamma,
                             void* hbuf, void* xq, float* xs, hipStream_t s) {
  if (fp8)
    norm_quant_kernel<true><<<T, NQ_THREADS, 0, s>>>(d, eps, x, gamma,
                                                     static_cast<uint16_t*>(hbuf), xq, xs);
  else
    norm_quant_kernel<false><<<T, NQ_THREADS, 0, s>>>(d, eps, x, gamma, nullptr, xq, nullptr);
  return hipGetLastError();
}

hipError_t launch_router_gemm_bf16(int T, int d, int E, int ksplit, const uint16_t* h,
                                   const uint16_t* wr, float* zpart, hipStream_t s) {
  dim3 grid((T + 63) / 64, (E + RG_E - 1) / RG_E, ksplit);
  router_gemm_bf16_kernel<<<grid, 256, 0, s>>>(T, d, E, d / ksplit, h, wr, zpart);
  return hipGetLastError();
}

hipError_t launch_router_gemm_f32(int T, int d, int E, const float* h, const float* wr,
                                  float* zpart, hipStream_t s) {
  const long n = (long)T * E;
  router_gemm_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(T, d, E, h, wr, zpart);
  return hipGetLastError();
}

hipError_t launch_topk(int T, int E, int k, int ksplit, float* zpart, const float* bias,
                       float scaling, int renorm, int32_t* ids, float* w, float* gap,
                       hipStream_t s) {
  const unsigned grid = (unsigned)((T + TK_WAVES - 1) / TK_WAVES);
  // with split-K partials, reduce them over all CUs first: one wave per token
  // summing ksplit partials of each expert is a long dependent load chain
  if (ksplit > 1) {
    const long n = (long)T * E;
    zsum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, ksplit, zpart);
    ksplit = 1;
  }
#define K2_TOPK(J, K)                                                                      \
  topk_kernel<J, K><<<grid, TK_WAVES * 64, 0, s>>>(T, E, k, ksplit, zpart, bias, scaling, \
                                                   renorm, ids, w, gap)
  if (E <= 64 && k <= 8) K2_TOPK(1, 8);
  else if (E <= 384 && k <= 8) K2_TOPK(6, 8);
  else if (E <= 1024 && k <= 32) K2_TOPK(16, 32);
  else return hipErrorInvalidValue;
#undef K2_TOPK
  return hipGetLastError();
}

hipError_t launch_dense_route(int T, float scaling, int32_t* ids, float* w, float* gap,
                              hipStream_t s) {
  dense_route_kernel<<<(T + 255) / 256, 256, 0, s>>>(T, scaling, ids, w, gap);
  return hipGetLastError();
}

}  // namespace k2
