// Shared device/host helpers for the gfx950 (CDNA4) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define QLS_DEV __device__ __forceinline__

// ---------------------------------------------------------------- bf16 bits
// bf16 <-> float through raw 16-bit patterns.  The float -> bf16 direction uses
// the hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
QLS_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
QLS_DEV uint32_t pack2_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
QLS_DEV uint16_t f2bf(float f) { return (uint16_t)(pack2_bf16(f, 0.f) & 0xFFFFu); }
QLS_DEV float bflo(uint32_t w) { return __uint_as_float(w << 16); }
QLS_DEV float bfhi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] B[16x32].  Lane l supplies
// row l%32 of A and column l%32 of B, eight consecutive contraction slots
// 8*(l/32)+j.  D: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
QLS_DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].  Lane l supplies
// row l%16 of A / column l%16 of B, contraction slots 8*(l/16)+j.  D: lane l
// holds column l%16, rows 4*(l/16) + i.
QLS_DEV f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- misc
QLS_DEV float warp_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
QLS_DEV float warp_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

static inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
