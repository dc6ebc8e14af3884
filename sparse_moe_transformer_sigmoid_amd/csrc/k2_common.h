// Device helpers shared by the gfx950 kernels of the K2 MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;
constexpr int QBLK = 128;          // FP8 block edge (weights 128x128, activations 1x128)
constexpr float FP8_MAX = 448.f;   // largest finite OCP e4m3 value

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Four fp32 values (already within +-448) -> four e4m3 codes, a in the low byte.
// gfx950's converter rounds to nearest even and produces OCP E4M3FN.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

__device__ __forceinline__ float clamp_fp8(float v) {
  return fminf(fmaxf(v, -FP8_MAX), FP8_MAX);
}

// Dynamic-quantisation scale of a block with absolute maximum `amax`.
__device__ __forceinline__ float fp8_scale(float amax) {
  return amax == 0.f ? 1.f : amax / FP8_MAX;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace k2
