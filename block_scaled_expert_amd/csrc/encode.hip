// Expert weight encoding and decoding on the GPU: bf16 / fp32 matrices to
// the canonical NVFP4 or MXFP8 layout with freshly computed scales, and back
// to fp32.  Weight sync re-encodes experts this way (Miles docs
// "inkling-2-small", section 5 on weight updates; the fp32 scale of NVFP4 is
// recomputed from the data on every encode), and the format definitions are
// those of the checkpoint (SGLang cookbook "Inkling-2-Small", section 2
// "Checkpoints"): NVFP4 = E2M1 codes, one E4M3 scale per 16 elements of a
// row and one fp32 scale per matrix; MXFP8 = E4M3 codes, one E8M0 scale per
// 32 elements of a row.
//
// Every floating-point step is one IEEE fp32 operation in the order the
// definition states (no contraction), so codes and scales are bit-identical
// to the definition.
#pragma clang fp contract(off)

#include "moe_common.h"
#include "launch.h"
#include "quant_row.h"

#include <algorithm>

namespace moe {

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Per-matrix max |w| as fp32 bits: |w| >= 0, so the bit patterns order like
// the values and an integer atomic maximum gives the same result in any
// order.  grid = (chunks, nmat); each workgroup reduces its chunk in LDS and
// adds one atomic, so a matrix's slot sees at most `chunks` of them.
template <typename InT>
__global__ __launch_bounds__(256) void k_amax(const InT* __restrict__ w, long per_mat, uint32_t* __restrict__ amax) {
  __shared__ float red[4];
  const int mat = blockIdx.y;
  const InT* m = w + (size_t)mat * per_mat;
  float a = 0.0f;
  const long stride = (long)gridDim.x * 256 * 16;
  for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 16; i < per_mat; i += stride) {
    float v[16];
    load_block<InT>(m + i, 16, v);
#pragma unroll
    for (int k = 0; k < 16; k++) a = fmaxf(a, fabsf(v[k]));
  }
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&amax[mat], f_bits(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// The fp32 scale of a matrix from its max |w| (amax 0: scale 1).
__device__ inline float nv_tensor_scale(float A) { return A == 0.0f ? 1.0f : __fdiv_rn(A, 2688.0f); }

// One thread per 16-element block of one row of one matrix.
template <typename InT>
__global__ __launch_bounds__(256) void k_encode_nvfp4(const InT* __restrict__ w, long nblocks, int cols,
                                                      long per_mat, const uint32_t* __restrict__ amax,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const long e0 = b * 16;                       // first element (matrices are contiguous)
  const int mat = (int)(e0 / per_mat);
  const float A = bits_f(amax[mat]);
  const float gs = nv_tensor_scale(A);
  float v[16];
  load_block<InT>(w + e0, 16, v);
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) ab = fmaxf(ab, fabsf(v[i]));
  uint32_t sc = e4m3_hw(__fdiv_rn(ab, __fmul_rn(6.0f, gs)));
  const float sigma = e4m3_decode(sc);
  uint32_t w0 = 0, w1 = 0;
  if (A != 0.0f && sigma != 0.0f) {
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
  if (A == 0.0f) sc = 0;
  *reinterpret_cast<uint2*>(codes + e0 / 2) = make_uint2(w0, w1);
  scales[b] = (uint8_t)sc;
}

// amax bits -> fp32 scale; matrix m's scale goes to
// gs[(m / group) * stride + m % group].
__global__ __launch_bounds__(256) void k_finish_gs(const uint32_t* __restrict__ amax, int nmat,
                                                   float* __restrict__ gs, int group, int stride) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= nmat) return;
  gs[(m / group) * stride + m % group] = nv_tensor_scale(bits_f(amax[m]));
}

// Decode: one thread per block (16 elements NVFP4, 32 MXFP8).
template <int FMT>
__global__ __launch_bounds__(256) void k_decode(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                const float* __restrict__ gs, long nblocks, long per_mat, int group,
                                                int stride, float* __restrict__ out) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  if (FMT == 1) {
    const long e0 = b * 16;
    const int mat = (int)(e0 / per_mat);
    const float g = gs[(mat / group) * stride + mat % group];
    const float sigma = e4m3_decode(scales[b]);
    const uint2 q = *reinterpret_cast<const uint2*>(codes + e0 / 2);
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const uint32_t c = ((i < 8 ? q.x : q.y) >> (4 * (i & 7))) & 15u;
      const uint32_t m = c & 7u;
      const float mag = m < 2 ? 0.5f * (float)m : (float)(2 + (m & 1)) * pow2f((int)(m >> 1) - 2);
      const float val = (c & 8u) ? -mag : mag;
      out[e0 + i] = __fmul_rn(__fmul_rn(val, sigma), g);   // val * sigma is exact
    }
  } else {
    const long e0 = b * 32;
    const int E = (int)scales[b] - 127;
#pragma unroll
    for (int i = 0; i < 32; i++) out[e0 + i] = ldexpf(e4m3_decode(codes[e0 + i]), E);
  }
}

int launch_encode_weights(int fmt, int dtype, const void* w, int nmat, int rows, int cols, uint8_t* codes,
                          uint8_t* scales, float* gs, int gs_group, int gs_stride, uint32_t* amax,
                          hipStream_t stream) {
  if (nmat <= 0 || rows <= 0) return 0;
  if (fmt == 2)
    return launch_quant(2, dtype, w, nmat * rows, nullptr, cols, codes, scales, nullptr, stream);
  const long per_mat = (long)rows * cols;
  hipLaunchKernelGGL(k_zero_u32, dim3(ceil_div(nmat, 256)), dim3(256), 0, stream, amax, nmat);
  const int chunks = (int)std::min<long>(ceil_div(per_mat, 256L * 16), 64L);
  const dim3 ga(chunks, nmat);
  if (dtype == 0)
    hipLaunchKernelGGL(k_amax<uint16_t>, ga, dim3(256), 0, stream, (const uint16_t*)w, per_mat, amax);
  else
    hipLaunchKernelGGL(k_amax<float>, ga, dim3(256), 0, stream, (const float*)w, per_mat, amax);
  const long nblocks = (long)nmat * per_mat / 16;
  const dim3 ge(ceil_div(nblocks, 256L));
  if (dtype == 0)
    hipLaunchKernelGGL(k_encode_nvfp4<uint16_t>, ge, dim3(256), 0, stream, (const uint16_t*)w, nblocks, cols,
                       per_mat, amax, codes, scales);
  else
    hipLaunchKernelGGL(k_encode_nvfp4<float>, ge, dim3(256), 0, stream, (const float*)w, nblocks, cols, per_mat,
                       amax, codes, scales);
  hipLaunchKernelGGL(k_finish_gs, dim3(ceil_div(nmat, 256)), dim3(256), 0, stream, amax, nmat, gs, gs_group,
                     gs_stride);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode_weights(int fmt, const uint8_t* codes, const uint8_t* scales, const float* gs, int nmat, int rows,
                          int cols, int gs_group, int gs_stride, float* out, hipStream_t stream) {
  if (nmat <= 0 || rows <= 0) return 0;
  const long per_mat = (long)rows * cols;
  const long nblocks = (long)nmat * per_mat / (fmt == 1 ? 16 : 32);
  const dim3 g(ceil_div(nblocks, 256L));
  if (fmt == 1)
    hipLaunchKernelGGL(k_decode<1>, g, dim3(256), 0, stream, codes, scales, gs, nblocks, per_mat, gs_group,
                       gs_stride, out);
  else
    hipLaunchKernelGGL(k_decode<2>, g, dim3(256), 0, stream, codes, scales, gs, nblocks, per_mat, 1, 0, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
