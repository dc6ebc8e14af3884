// Weighted combine + residual add, and the one-time FP8 weight re-layout.
//
// Combine ("Kimi-K2-Base", Mixture of experts: renormalised top-k weights
// times the routed scaling factor; "Kimi K2 · Dense transformer block", Code:
// residual add after the MLP): per token, in fp32 and in ascending expert
// order, y = sum_slot w * row + shared, then out = x + y rounded once.
#include "k2_common.h"
#include "k2_launch.h"

namespace k2 {

namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

template <bool XBF16, bool OUTF32>
__global__ __launch_bounds__(256) void combine_kernel(int T, int d, int k,
                                                     const float* __restrict__ rows,
                                                     const int32_t* __restrict__ pair_row,
                                                     const float* __restrict__ topk_w,
                                                     int mul_w, const float* __restrict__ shared,
                                                     const void* __restrict__ residual,
                                                     void* __restrict__ out) {
  // one token per blockIdx.x, 1024 columns per blockIdx.y: small batches
  // still spread over the chip, and the k row reads of a thread are issued
  // together (the sum itself stays in slot order).  Expert rows and the
  // shared output are read once and the output written once: non-temporal.
  const int t = blockIdx.x;
  const int P = T * k;
  const int d4 = d >> 2;
  const int n4 = blockIdx.y * 256 + threadIdx.x;
  if (n4 < d4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int slot = 0; slot < k; ++slot) {
      const int p = t * k + slot;
      const int r = min(max(pair_row[p], 0), P - 1);
      float4 v = load_nt(reinterpret_cast<const float4*>(rows + (size_t)r * d) + n4);
      if (mul_w) {
        const float w = topk_w[p];
        // rounded products, as the fused path stores them (no fma contraction)
        v.x = __fmul_rn(v.x, w); v.y = __fmul_rn(v.y, w);
        v.z = __fmul_rn(v.z, w); v.w = __fmul_rn(v.w, w);
      }
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (shared) {
      const float4 v = load_nt(reinterpret_cast<const float4*>(shared + (size_t)t * d) + n4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (residual) {
      if constexpr (XBF16) {
        const uint2 xb = reinterpret_cast<const uint2*>(
            static_cast<const uint16_t*>(residual) + (size_t)t * d)[n4];
        acc.x = bf16_to_f32(xb.x & 0xFFFFu) + acc.x;
        acc.y = bf16_to_f32(xb.x >> 16) + acc.y;
        acc.z = bf16_to_f32(xb.y & 0xFFFFu) + acc.z;
        acc.w = bf16_to_f32(xb.y >> 16) + acc.w;
      } else {
        const float4 xv = reinterpret_cast<const float4*>(
            static_cast<const float*>(residual) + (size_t)t * d)[n4];
        acc.x = xv.x + acc.x; acc.y = xv.y + acc.y; acc.z = xv.z + acc.z; acc.w = xv.w + acc.w;
      }
    }
    if constexpr (OUTF32) {
      f4v* o = reinterpret_cast<f4v*>(static_cast<float*>(out) + (size_t)t * d) + n4;
      __builtin_nontemporal_store(f4v{acc.x, acc.y, acc.z, acc.w}, o);
    } else {
      const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
      u2v* o = reinterpret_cast<u2v*>(static_cast<uint16_t*>(out) + (size_t)t * d) + n4;
      __builtin_nontemporal_store(u2v{lo, hi}, o);
    }
  }
}

// One thread per 16-byte piece of the packed codes of one expert.
// Gate/up: [chunk j][wave w][kb][rt][half p][lane][16 B]; rt 0,1 = gate
// hidden 128j + 32w + 16rt + lane%16, rt 2,3 = up rows of the same hidden.
// Down: [chunk j][wave w][kb][rt][p][lane][16 B], output row
// 256j + 64w + 16rt + lane%16.  Columns: kb*128 + 32*(lane/16) + 16p.
__global__ __launch_bounds__(256) void pack_fp8_kernel(int d, int I,
                                                      const uint8_t* __restrict__ wg,
                                                      const uint8_t* __restrict__ wu,
                                                      const uint8_t* __restrict__ wd,
                                                      uint8_t* __restrict__ dst) {
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  const long n_gu = 2L * I * d / 16, n_dn = (long)d * I / 16;
  if (q >= n_gu + n_dn) return;
  const uint8_t* src;
  if (q < n_gu) {
    const int lane = q & 63, p = (q >> 6) & 1, rt = (q >> 7) & 3;
    long rest = q >> 9;
    const int nkb = d / QBLK;
    const int kb = (int)(rest % nkb);
    rest /= nkb;
    const int w = (int)(rest & 3), j = (int)(rest >> 2);
    const int hidden = j * 128 + 32 * w + 16 * (rt & 1) + (lane & 15);
    src = (rt < 2 ? wg : wu) + (size_t)hidden * d + kb * 128 + (lane >> 4) * 32 + p * 16;
  } else {
    const long q2 = q - n_gu;
    const int lane = q2 & 63, p = (q2 >> 6) & 1, rt = (q2 >> 7) & 3;
    long rest = q2 >> 9;
    const int nkb = I / QBLK;
    const int kb = (int)(rest % nkb);
    rest /= nkb;
    const int w = (int)(rest & 3), j = (int)(rest >> 2);
    const int row = j * 256 + 64 * w + 16 * rt + (lane & 15);
    src = wd + (size_t)row * I + kb * 128 + (lane >> 4) * 32 + p * 16;
  }
  reinterpret_cast<uint4*>(dst)[q] = *reinterpret_cast<const uint4*>(src);
}

// gate/up scales interleaved as [j][kb][gate, up]; down scales copied as is.
__global__ void pack_scales_kernel(int nb_gu, int nb_dn, const float* __restrict__ sg,
                                   const float* __restrict__ su, const float* __restrict__ sd,
                                   float* __restrict__ dgu, float* __restrict__ ddn) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nb_gu) {
    dgu[2 * i] = sg[i];
    dgu[2 * i + 1] = su[i];
  }
  if (i < nb_dn) ddn[i] = sd[i];
}

}  // namespace

hipError_t launch_combine(bool x_bf16, bool out_f32, int T, int d, int k, const float* rows,
                          const int32_t* pair_row, const float* topk_w, int mul_w,
                          const float* shared_out, const void* residual, void* out,
                          hipStream_t s) {
#define K2_COMB(XB, OF)                                                                   \
  combine_kernel<XB, OF><<<dim3(T, (d / 4 + 255) / 256), 256, 0, s>>>(                     \
      T, d, k, rows, pair_row, topk_w, mul_w, shared_out, residual, out)
  if (x_bf16) {
    if (out_f32) K2_COMB(true, true); else K2_COMB(true, false);
  } else {
    K2_COMB(false, true);
  }
#undef K2_COMB
  return hipGetLastError();
}

hipError_t launch_pack_fp8(int d, int I, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                           const float* sg, const float* su, const float* sd, uint8_t* dst_codes,
                           float* dst_gu_scales, float* dst_d_scales, hipStream_t s) {
  const long n = 3L * I * d / 16;
  pack_fp8_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(d, I, wg, wu, wd, dst_codes);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nb = (I / QBLK) * (d / QBLK);
  pack_scales_kernel<<<(nb + 255) / 256, 256, 0, s>>>(nb, nb, sg, su, sd, dst_gu_scales,
                                                      dst_d_scales);
  return hipGetLastError();
}

}  // namespace k2
