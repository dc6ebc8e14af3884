// Device helpers shared by the MLA kernels (mla.hip, mla_mha.hip): the
// latent and head widths of Kimi K2's attention ("Kimi K2 · Architecture",
// config.json: kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128,
// v_head_dim 128), bf16 packing and high/low splits, the bf16 MFMA, rotary
// pairs, and direct global -> LDS copies.
#pragma once
#include <math.h>

#include "k2_common.h"

namespace k2 {

namespace {

constexpr int DL = 512;           // latent width (kv_lora)
constexpr int DR = 64;            // rotary width
constexpr int DQ = DL + DR;       // absorbed query / cache row width
constexpr int DN = 128;           // query/key features without position (qk_nope)
constexpr int DV = 128;           // value features (v_head)

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)f32_to_bf16_rne(f); }

__device__ __forceinline__ __bf16 to_bf16(float f) {
  return __builtin_bit_cast(__bf16, bf16_bits(f));
}

// e4m3 code -> float (exact)
__device__ __forceinline__ float e4m3_val(uint32_t code) {
  const v2f p = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false);
  return p[0];
}

__device__ __forceinline__ int token_pos(const int32_t* cached_len, int t, int n_new,
                                        int max_len, int* seq) {
  *seq = t / n_new;
  const int p = cached_len[*seq] + t % n_new;
  return min(max(p, 0), max_len - 1);
}

// rotate (a, b) by the angle with cosine cs and sine sn in double, round to fp32
__device__ __forceinline__ void rope_apply(float a, float b, double cs, double sn, float* ra,
                                           float* rb) {
  *ra = (float)((double)a * cs - (double)b * sn);
  *rb = (float)((double)a * sn + (double)b * cs);
}

// rotate (a, b) by pos * f in double, round to fp32
__device__ __forceinline__ void rope_pair(float a, float b, int pos, double f, float* ra,
                                          float* rb) {
  double sn, cs;
  sincos((double)pos * f, &sn, &cs);
  rope_apply(a, b, cs, sn, ra, rb);
}

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two fp32 values -> packed bf16 (a low), round to nearest even (gfx950's
// converter)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}
// the bf16 high parts of (a, b) (lo = 0) or the bf16 roundings of their
// remainders a - high (lo = 1; exact in fp32), packed
__device__ __forceinline__ uint32_t bf16_half2(float a, float b, float lo) {
  const uint32_t hb = pack_bf16(a, b);
  return pack_bf16(fmaf(-lo, __uint_as_float(hb << 16), a),
                   fmaf(-lo, __uint_as_float(hb & 0xFFFF0000u), b));
}

// Direct global -> LDS copies (global_load_lds_dword / _dwordx4): lane l's 4
// or 16 bytes from global [base + voff] land at LDS byte address M0 + l *
// size.  They complete in issue order with the other vector loads (vmcnt);
// the compiler does not track them, so the kernel waits for them itself.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
// wait until at most n (wave-uniform, 0..9) of this wave's vector loads are
// outstanding
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" : : : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" : : : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" : : : "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" : : : "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" : : : "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" : : : "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" : : : "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" : : : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(9)" : : : "memory"); break;
  }
}

// eight fp32 values -> their bf16 high parts (hi) and remainder roundings (lo)
__device__ __forceinline__ void split8(const float4 a, const float4 b, v8bf* hi, v8bf* lo) {
  const uint4 h = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y),
                             pack_bf16(b.z, b.w));
  *hi = __builtin_bit_cast(v8bf, h);
  *lo = __builtin_bit_cast(v8bf, make_uint4(bf16_half2(a.x, a.y, 1.f), bf16_half2(a.z, a.w, 1.f),
                                            bf16_half2(b.x, b.y, 1.f), bf16_half2(b.z, b.w, 1.f)));
}

}  // namespace

}  // namespace k2
