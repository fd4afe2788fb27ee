// Internal helpers shared by the gfx950 kernels of the MoE library.
//
// Element formats (OCP MX / NVFP4 conventions that the pages' "NVFP4" and
// "MXFP8" name; SGLang cookbook "Inkling-2-Small", section 2 "Checkpoints"):
//   E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; max 6.
//   E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa; max 448; the
//         all-ones magnitude is NaN and is never produced.
//   E8M0: 2^(c-127).
// Conversions round to nearest, ties to the even code, saturate to the
// largest finite magnitude and keep the sign of zero; a NaN encodes as +0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's uint4 is a struct whose copies can end up
// in scratch memory)
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__host__ __device__ inline float bits_f(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}
__host__ __device__ inline uint32_t f_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}
// 2^e as fp32 for e in [-126, 127].
__host__ __device__ inline float pow2f(int e) { return bits_f((uint32_t)(e + 127) << 23); }

// fp32 -> E4M3 code.  For |x| < 448 the magnitude is rounded on the grid of
// its binade (2^(e-3), e = max(floor(log2|x|), -6)); the integer quotient's
// parity is the code's parity, so rint's ties-to-even is the code's.
__host__ __device__ inline uint32_t e4m3_encode(float x) {
  const uint32_t b = f_bits(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return 0u;
  if (a >= 448.0f) return sign | 0x7Eu;
  int e = (int)((b >> 23) & 0xFFu) - 127;
  e = e < -6 ? -6 : e;
  const float q = rintf(a * pow2f(3 - e));
  return sign | (uint32_t)((e + 7) * 8 + (int)q - 8);
}

__host__ __device__ inline float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float mag = e == 0 ? (float)m * pow2f(-9) : (float)(8u + m) * pow2f((int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

// fp32 -> E2M1 code (same construction on the E2M1 grid).
__host__ __device__ inline uint32_t e2m1_encode(float x) {
  const uint32_t b = f_bits(x);
  const uint32_t sign = (b >> 28) & 0x8u;
  const float a = fabsf(x);
  if (!(a == a)) return 0u;
  if (a >= 6.0f) return sign | 7u;
  int e = (int)((b >> 23) & 0xFFu) - 127;
  e = e < 0 ? 0 : e;
  const float q = rintf(a * pow2f(1 - e));
  return sign | (uint32_t)((e + 1) * 2 + (int)q - 2);
}

// E8M0 exponent E for an MX block of 32 with max magnitude amax (E4M3
// elements, emax 8): E = clamp(floor(log2 amax) - 8, -127, 127); -127 for a
// zero block.  Subnormal amax has floor(log2) <= -127, so it clamps too.
__host__ __device__ inline int mx_exponent(float amax) {
  const uint32_t ef = (f_bits(amax) >> 23) & 0xFFu;
  if (ef == 0) return -127;
  const int e = (int)ef - 127 - 8;
  return e < -127 ? -127 : e;
}

// gfx950's conversion instructions (v_cvt_scalef32_pk_fp8_f32,
// v_cvt_scalef32_pk_fp4_f32, scale 1.0) give the same codes as the encoders
// above for every finite input: checked on the device over every finite
// bf16 pattern, 4M random fp32 values, each grid's rounding midpoints and
// their neighbours, and the saturation edges.  Both round to nearest even.
// The E2M1 conversion saturates (+-inf too) but sends NaN to +-6; the E4M3
// conversion does not saturate (above 448 and at +-inf it gives the NaN
// code), so its input is clamped to +-448, NaN to 0 -- what e4m3_encode does.
typedef short v2s __attribute__((ext_vector_type(2)));
__device__ inline float clamp448(float x) { return x == x ? fminf(fmaxf(x, -448.0f), 448.0f) : 0.0f; }
__device__ inline uint32_t e4m3_hw(float x) {
  const float c = clamp448(x);
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, c, c, 1.0f, false);
  return (uint32_t)(uint16_t)r[0] & 0xFFu;
}
// four E4M3 codes, a in the low byte
__device__ inline uint32_t e4m3_pack4(float a, float b, float c, float d) {
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, clamp448(a), clamp448(b), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, clamp448(c), clamp448(d), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}
// eight E2M1 codes of v[i] * r (each product rounded once), v[0] in the low
// nibble.  For finite v and finite r no product is NaN; callers whose r can
// overflow to inf take e2m1_encode there (0 * inf is NaN, which it sends to 0).
__device__ inline uint32_t e2m1_pack8(const float* v, float r) {
#pragma clang fp contract(off)
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[0], r), __fmul_rn(v[1], r), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[2], r), __fmul_rn(v[3], r), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[4], r), __fmul_rn(v[5], r), 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[6], r), __fmul_rn(v[7], r), 1.0f, 3);
  return w;
}

// One MXFP8 element given its block's step 2^-E (E = mx_exponent(amax)):
// the scaling is exact, the encode rounds once.
__device__ inline uint32_t mx_encode(float v, float step) { return e4m3_hw(__fmul_rn(v, step)); }

// Workgroup barrier for hand-offs through LDS: waits for the wave's own LDS
// operations, then for every wave.  HIP's __syncthreads also waits for all
// of the wave's outstanding global loads, which in a k loop that prefetches
// the next step through registers stalls every step for a full memory round
// trip; here those loads stay in flight (the compiler waits for each at its
// first use).
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline float bf16_to_f32(uint16_t h) { return bits_f((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = f_bits(f);
  const uint32_t r = b + 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Two fp32 scale factors applied together: v * a * b as
// ldexp(v * (mant(a) * mant(b)), exp(a) + exp(b)), mant in [0.5, 1).  A
// token's activation scale and an expert's weight scale can each lie far
// outside the range of their product with v (a row of 2^60-sized values has
// an NVFP4 scale near 2^50), so multiplying them in one after the other can
// overflow or underflow on the way; here only the final result can.  Two
// roundings, like the two products it replaces; frexp / ldexp are single
// instructions.
struct ScalePair {
  float m;
  int e;
};
__device__ inline ScalePair split_scale(float a) {
  return ScalePair{__builtin_amdgcn_frexp_mantf(a), __builtin_amdgcn_frexp_expf(a)};
}
__device__ inline ScalePair operator*(ScalePair a, ScalePair b) { return ScalePair{a.m * b.m, a.e + b.e}; }
__device__ inline float apply_scale(float v, ScalePair s) { return __builtin_amdgcn_ldexpf(v * s.m, s.e); }

// Reciprocal from the hardware instruction (v_rcp_f32, within 1 ulp; 1/inf
// is 0).  The epilogues take their quotients this way: an IEEE division
// expands to about ten instructions, which in the large-M gate/up epilogue
// was as much vector-ALU work as the k loop's operand expansion.
__device__ inline float rcp_fast(float y) { return __builtin_amdgcn_rcpf(y); }

// tanh from one hardware exponential: tanh|x| = 1 - 2 / (e^{2|x|} + 1)
// (e^{2|x|} = inf gives exactly 1).  That difference cancels as |x| -> 0
// (its relative error grows like 1e-7 / |x|), so below |x| = 1/8 the odd
// Taylor series to x^7 is used instead (truncation below 2e-9 relative).
// Relative error: below about 2e-6 everywhere, measured against float64.
__device__ inline float tanh_fast(float x) {
  const float a = fabsf(x);
  const float e = __expf(2.0f * a);
  const float big = 1.0f - 2.0f * rcp_fast(e + 1.0f);
  const float a2 = a * a;
  const float small = a * (1.0f + a2 * (-1.0f / 3.0f + a2 * (2.0f / 15.0f + a2 * (-17.0f / 315.0f))));
  return copysignf(a < 0.125f ? small : big, x);
}

// Cap + SwiGLU on fp32 gate/up values (cap forms of enum moe_cap_form).
__device__ inline float cap_swiglu(float g, float u, int form, float c, float inv_c) {
  if (form == 0) {            // soft cap on gate and up
    g = c * tanh_fast(g * inv_c);
    u = c * tanh_fast(u * inv_c);
  } else if (form == 1) {     // hard cap
    g = fminf(g, c);
    u = fminf(fmaxf(u, -c), c);
  }
  float h = g * rcp_fast(1.0f + __expf(-g)) * u;
  if (form == 2) h = c * tanh_fast(h * inv_c);
  return h;
}

// The same on N pairs in place (g[i] <- h[i]), the arithmetic of cap_swiglu
// per element.  Each form's work sits in its own loop under one uniform
// branch: with the branch per element the compiler evaluates every form and
// selects.
template <int N>
__device__ inline void cap_swiglu_n(float (&g)[N], float (&u)[N], int form, float c, float inv_c) {
  if (form == 0) {
#pragma unroll
    for (int i = 0; i < N; i++) {
      g[i] = c * tanh_fast(g[i] * inv_c);
      u[i] = c * tanh_fast(u[i] * inv_c);
    }
  } else if (form == 1) {
#pragma unroll
    for (int i = 0; i < N; i++) {
      g[i] = fminf(g[i], c);
      u[i] = fminf(fmaxf(u[i], -c), c);
    }
  }
#pragma unroll
  for (int i = 0; i < N; i++) g[i] = g[i] * rcp_fast(1.0f + __expf(-g[i])) * u[i];
  if (form == 2) {
#pragma unroll
    for (int i = 0; i < N; i++) g[i] = c * tanh_fast(g[i] * inv_c);
  }
}

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
