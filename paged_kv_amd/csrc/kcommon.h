// Device-side helpers shared by the HIP kernels of libattnq (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define ATTNQ_DEV __device__ __forceinline__

namespace attnq {

// Native vector types (HIP's uint4 is a union-wrapped struct that register
// promotion does not always see through).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- 16-bit floats
ATTNQ_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

ATTNQ_DEV uint32_t f32_to_bf16(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

ATTNQ_DEV float f16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

ATTNQ_DEV uint32_t f32_to_f16(float f) {  // hardware conversion, round to nearest even
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// 16-bit storage value -> fp32, `is_bf16` selects the format.
ATTNQ_DEV float h16_to_f32(uint32_t bits16, bool is_bf16) {
  return is_bf16 ? bf16_to_f32(bits16) : f16_to_f32(bits16);
}
ATTNQ_DEV uint32_t f32_to_h16(float f, bool is_bf16) {
  return is_bf16 ? f32_to_bf16(f) : f32_to_f16(f);
}

// ---------------------------------------------------------------- fp8 e4m3fn
// Encode v (already divided by its scale): NaN -> 0x7F, |v| clamped to 448,
// round to nearest even on the e4m3 grid, sign kept (-0 and negative values
// that round to zero give 0x80).
ATTNQ_DEV uint32_t e4m3fn_encode(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fu;
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __uint_as_float(u & 0x7fffffffu);
  a = a > 448.0f ? 448.0f : a;
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: fixed quantum 2^-9, codes 0..8
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {  // keep 3 fraction bits with round-to-nearest-even, re-bias 127 -> 7
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
  }
  return code | sign;
}

// e4m3fn code -> fp16 bit pattern of (value * 2^-8), exact for every finite
// code: the 7 magnitude bits land on fp16's exponent/fraction so that
// fp16(e + 8 - 15 ... ) absorbs the bias difference as a 2^-8 factor.
ATTNQ_DEV uint32_t e4m3_to_f16_scaled(uint32_t code) {
  return ((code & 0x80u) << 8) | ((code & 0x7fu) << 7);
}

// Four fp8 codes packed in a dword -> two dwords of fp16 pairs (value * 2^-8).
ATTNQ_DEV void e4m3x4_to_f16x4_scaled(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // place byte k at the high byte of 16-bit lane k: lo = [b1 b0] -> 0xb1 00 b0 00
  uint32_t l = __builtin_amdgcn_perm(0u, w, 0x010c000cu);  // bytes: [0]=0,[1]=b0,[2]=0,[3]=b1
  uint32_t h = __builtin_amdgcn_perm(0u, w, 0x030c020cu);
  lo = ((l >> 1) & 0x3f803f80u) | (l & 0x80008000u);
  hi = ((h >> 1) & 0x3f803f80u) | (h & 0x80008000u);
}

// x / s correctly rounded, from r = 1/s (itself correctly rounded) in three
// operations: q0 = x r, e = x - q0 s (exact through the fused multiply-add),
// q = q0 + e r (Markstein's correction), with the sign of x kept for -0.
// Equal to the IEEE quotient whenever it is a normal number; where the
// quotient is subnormal it may differ in its last bits only, which no int8
// or e4m3fn code can see.  Valid for s >= 1e-30 (1/s finite); callers use the
// plain division below that.
ATTNQ_DEV float quot_by_recip(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}
constexpr float QUOT_MIN_SCALE = 1e-30f;

// The same quotient without the sign fix-up of a zero result, for int8 codes:
// rint(+0) and rint(-0) give the same code.
ATTNQ_DEV float quot_by_recip_i8(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e, r, q0);
}

// rint(v) (ties to even) clamped to [-127, 127]; NaN -> 0.  v_cvt_i32_f32
// saturates out-of-range values and maps NaN to 0, so one integer clamp
// after it finishes the job (a C cast of NaN or of an out-of-range float
// would be undefined).
ATTNQ_DEV int32_t int8_encode(float v) {
  int32_t i;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(__builtin_rintf(v)));
  return i > 127 ? 127 : (i < -127 ? -127 : i);
}

// ---------------------------------------------------------------- reductions
ATTNQ_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

ATTNQ_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).  Keeps
// register-array indices constant where #pragma unroll is not honoured.
template <int B, int E, typename F>
ATTNQ_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace attnq
