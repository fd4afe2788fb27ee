// Per-row activation quantization bodies, shared by the quantization kernels
// and the small-batch fused quantize + dispatch launch.  Formats: W4A4 /
// W8A8 (Miles docs "inkling-2-small" section 5.3); the NVFP4 fp32 scale spans
// each row's full width (SGLang cookbook "Inkling-2-Small" section 2,
// "Parallelism").
//
// A group of 256 threads quantizes one row; threads take whole scale blocks
// (16 elements for NVFP4, 32 for MXFP8), so loads are contiguous runs across
// the wave.  Every floating-point step is a single IEEE fp32 operation in the
// order the format definition states (no contraction), so codes and scales
// are bit-identical to the definition.
#pragma once

#include "moe_common.h"

namespace moe {

template <typename InT>
__device__ inline void load_block(const InT* p, int n, float* v);

template <>
__device__ inline void load_block<uint16_t>(const uint16_t* p, int n, float* v) {
  const v4u* q = reinterpret_cast<const v4u*>(p);
  for (int i = 0; i < n / 8; i++) {
    const v4u w = q[i];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[8 * i + 2 * j] = bits_f(w[j] << 16);
      v[8 * i + 2 * j + 1] = bits_f(w[j] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ inline void load_block<float>(const float* p, int n, float* v) {
  const v4f* q = reinterpret_cast<const v4f*>(p);
  for (int i = 0; i < n / 4; i++) {
    const v4f w = q[i];
    v[4 * i] = w.x;
    v[4 * i + 1] = w.y;
    v[4 * i + 2] = w.z;
    v[4 * i + 3] = w.w;
  }
}

// Maximum over a group of 256 threads (4 waves; t = thread in the group),
// through 4 floats of LDS.  Contains a workgroup barrier: every thread of
// the workgroup must call it.
__device__ inline float group_max(float v, float* red, int t) {
  v = wave_max(v);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One NVFP4 block of 16 values of a row with fp32 scale gs (denom = 6 gs):
// returns its E4M3 scale byte, codes in w0 (values 0-7) and w1 (8-15).
__device__ inline uint32_t nvfp4_block(const float* v, float gs, float denom, bool zero_row, uint32_t& w0,
                                       uint32_t& w1) {
#pragma clang fp contract(off)
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) ab = fmaxf(ab, fabsf(v[i]));
  uint32_t sc = e4m3_hw(__fdiv_rn(ab, denom));
  const float sigma = e4m3_decode(sc);
  w0 = 0;
  w1 = 0;
  if (!zero_row && sigma != 0.0f) {
    const float r = __fdiv_rn(1.0f, __fmul_rn(sigma, gs));
    if (r <= 3.4028235e38f) {   // r overflows only where the row (or matrix) maximum is below ~4e-33
      w0 = e2m1_pack8(v, r);
      w1 = e2m1_pack8(v + 8, r);
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) w0 |= e2m1_encode(__fmul_rn(v[i], r)) << (4 * i);
#pragma unroll
      for (int i = 0; i < 8; i++) w1 |= e2m1_encode(__fmul_rn(v[8 + i], r)) << (4 * i);
    }
  }
  return zero_row ? 0u : sc;
}

// Where an NVFP4 row takes its fp32 scale (enum moe_act_gs): computed from
// the row (GS_ROW), read from one device word shared by the whole tensor
// (GS_TENSOR, written by k_act_gs_finish), or a kernel argument (GS_STATIC).
constexpr int GS_ROW = 0, GS_TENSOR = 1, GS_STATIC = 2;

// fp32 scale of an NVFP4 scale domain with maximum A: A / 2688 (one IEEE
// fp32 division; 2688 = 6 * 448), 1 for an all-zero domain.
__device__ inline float nvfp4_gs(float A) { return A == 0.0f ? 1.0f : __fdiv_rn(A, 2688.0f); }

// NVFP4 row of `cols` elements: codes (cols/2 bytes), E4M3 block scales
// (cols/16) and the fp32 row scale.  live == false: the row is read and the
// barrier taken, nothing is written.  MODE GS_ROW takes the row's own scale
// (and a workgroup barrier: every thread must call it); GS_TENSOR reads
// *gs_in; GS_STATIC uses gs_val (no barrier in either).
template <typename InT, int MODE = GS_ROW>
__device__ inline void quant_row_nvfp4(const InT* __restrict__ xr, int cols, int t, float* red, bool live,
                                       uint8_t* __restrict__ cr, uint8_t* __restrict__ sr,
                                       float* __restrict__ gs_out, const float* gs_in = nullptr,
                                       float gs_val = 1.0f) {
#pragma clang fp contract(off)
  const int nblk = cols / 16;
  bool zero_row = false;
  float gs;
  if constexpr (MODE == GS_ROW) {
    float A = 0.0f;
    for (int b = t; b < nblk; b += 256) {
      float v[16];
      load_block<InT>(xr + 16 * b, 16, v);
#pragma unroll
      for (int i = 0; i < 16; i++) A = fmaxf(A, fabsf(v[i]));
    }
    A = group_max(A, red, t);
    zero_row = (A == 0.0f);
    gs = nvfp4_gs(A);
  } else if constexpr (MODE == GS_TENSOR) {
    gs = *gs_in;
  } else {
    gs = gs_val;
  }
  const float denom = __fmul_rn(6.0f, gs);
  if (t == 0 && live) *gs_out = gs;

  for (int b = t; b < nblk; b += 256) {
    float v[16];
    load_block<InT>(xr + 16 * b, 16, v);
    uint32_t w0, w1;
    const uint32_t sc = nvfp4_block(v, gs, denom, zero_row, w0, w1);
    if (live) {
      *reinterpret_cast<uint2*>(cr + 8 * b) = make_uint2(w0, w1);
      sr[b] = (uint8_t)sc;
    }
  }
}

// The same NVFP4 row quantization by one wave (64 lanes, lane index t) with
// no workgroup barrier: several rows quantize side by side, one per wave.
// Outputs are device-scope stores (written through for readers on other
// XCDs).
template <typename InT>
__device__ inline void quant_row_nvfp4_wave(const InT* __restrict__ xr, int cols, int t,
                                            uint8_t* __restrict__ cr, uint8_t* __restrict__ sr,
                                            float* __restrict__ gs_out) {
#pragma clang fp contract(off)
  const int nblk = cols / 16;
  float A = 0.0f;
  for (int b = t; b < nblk; b += 64) {
    float v[16];
    load_block<InT>(xr + 16 * b, 16, v);
#pragma unroll
    for (int i = 0; i < 16; i++) A = fmaxf(A, fabsf(v[i]));
  }
  A = wave_max(A);
  const bool zero_row = (A == 0.0f);
  const float gs = zero_row ? 1.0f : __fdiv_rn(A, 2688.0f);
  const float denom = __fmul_rn(6.0f, gs);
  if (t == 0) __hip_atomic_store(gs_out, gs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int b = t; b < nblk; b += 64) {
    float v[16];
    load_block<InT>(xr + 16 * b, 16, v);
    uint32_t w0, w1;
    const uint32_t sc = nvfp4_block(v, gs, denom, zero_row, w0, w1);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(cr + 8 * b), (uint64_t)w0 | ((uint64_t)w1 << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sr + b, (uint8_t)sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// MXFP8 row: codes (cols bytes) and E8M0 block scales (cols/32).
template <typename InT>
__device__ inline void quant_row_mxfp8(const InT* __restrict__ xr, int cols, int t, bool live,
                                       uint8_t* __restrict__ cr, uint8_t* __restrict__ sr) {
#pragma clang fp contract(off)
  const int nblk = cols / 32;
  for (int b = t; b < nblk; b += 256) {
    float v[32];
    load_block<InT>(xr + 32 * b, 32, v);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) am = fmaxf(am, fabsf(v[i]));
    const int E = mx_exponent(am);
    const float step = pow2f(-E);   // -E in [-119, 127]
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; j++)
      w[j] = e4m3_pack4(__fmul_rn(v[4 * j], step), __fmul_rn(v[4 * j + 1], step), __fmul_rn(v[4 * j + 2], step),
                        __fmul_rn(v[4 * j + 3], step));
    if (live) {
      v4u* dst = reinterpret_cast<v4u*>(cr + 32 * b);
      dst[0] = v4u{w[0], w[1], w[2], w[3]};
      dst[1] = v4u{w[4], w[5], w[6], w[7]};
      sr[b] = (uint8_t)(E + 127);
    }
  }
}

}  // namespace moe
