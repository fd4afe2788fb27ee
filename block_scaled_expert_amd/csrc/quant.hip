// Per-row activation quantization (W4A4 / W8A8: Miles docs "inkling-2-small"
// section 5.3; the NVFP4 fp32 scale spans each row's full width: SGLang
// cookbook "Inkling-2-Small" section 2, "Parallelism").
//
// One workgroup per row; threads take whole scale blocks (16 elements for
// NVFP4, 32 for MXFP8), so loads are contiguous 32/64-byte runs across the
// wave.  HBM-bound: every input byte is read once from HBM (the NVFP4 second
// pass hits the cache) and every output byte written once.
//
// Every floating-point step is a single IEEE fp32 operation in the order the
// format definition states (no contraction), so codes and scales are
// bit-identical to the definition.
#pragma clang fp contract(off)

#include "moe_common.h"
#include "launch.h"

namespace moe {

template <typename InT>
__device__ inline void load_block(const InT* p, int n, float* v);

template <>
__device__ inline void load_block<uint16_t>(const uint16_t* p, int n, float* v) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  for (int i = 0; i < n / 8; i++) {
    const uint4 w = q[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[8 * i + 2 * j] = bits_f(ws[j] << 16);
      v[8 * i + 2 * j + 1] = bits_f(ws[j] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ inline void load_block<float>(const float* p, int n, float* v) {
  const float4* q = reinterpret_cast<const float4*>(p);
  for (int i = 0; i < n / 4; i++) {
    const float4 w = q[i];
    v[4 * i] = w.x;
    v[4 * i + 1] = w.y;
    v[4 * i + 2] = w.z;
    v[4 * i + 3] = w.w;
  }
}

// Row amax across the workgroup (256 threads = 4 waves).
__device__ inline float block_max(float v, float* lds) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
}

// NVFP4 rows: one workgroup per row, one 16-element block per thread and
// pass.  rows_dev (nullable): device row count that further limits rows.
template <typename InT>
__global__ __launch_bounds__(256) void k_quant_nvfp4(const InT* __restrict__ x, int rows,
                                                     const int* __restrict__ rows_dev, int cols,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     float* __restrict__ gs_out) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  int nrows = rows;
  if (rows_dev != nullptr) nrows = min(nrows, *rows_dev);
  if (row >= nrows) return;
  const InT* xr = x + (size_t)row * cols;
  const int nblk = cols / 16;

  float A = 0.0f;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    float v[16];
    load_block<InT>(xr + 16 * b, 16, v);
#pragma unroll
    for (int i = 0; i < 16; i++) A = fmaxf(A, fabsf(v[i]));
  }
  A = block_max(A, red);
  const bool zero_row = (A == 0.0f);
  const float gs = zero_row ? 1.0f : __fdiv_rn(A, 2688.0f);
  const float denom = __fmul_rn(6.0f, gs);
  if (threadIdx.x == 0) gs_out[row] = gs;

  uint8_t* cr = codes + (size_t)row * (cols / 2);
  uint8_t* sr = scales + (size_t)row * nblk;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    float v[16];
    load_block<InT>(xr + 16 * b, 16, v);
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) ab = fmaxf(ab, fabsf(v[i]));
    uint32_t sc = e4m3_encode(__fdiv_rn(ab, denom));
    const float sigma = e4m3_decode(sc);
    uint32_t w0 = 0, w1 = 0;
    if (!zero_row && sigma != 0.0f) {
      const float r = __fdiv_rn(1.0f, __fmul_rn(sigma, gs));
#pragma unroll
      for (int i = 0; i < 8; i++) w0 |= e2m1_encode(__fmul_rn(v[i], r)) << (4 * i);
#pragma unroll
      for (int i = 0; i < 8; i++) w1 |= e2m1_encode(__fmul_rn(v[8 + i], r)) << (4 * i);
    }
    if (zero_row) sc = 0;
    *reinterpret_cast<uint2*>(cr + 8 * b) = make_uint2(w0, w1);
    sr[b] = (uint8_t)sc;
  }
}

// MXFP8 rows: one workgroup per row, one 32-element block per thread and pass.
template <typename InT>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const InT* __restrict__ x, int rows,
                                                     const int* __restrict__ rows_dev, int cols,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int row = blockIdx.x;
  int nrows = rows;
  if (rows_dev != nullptr) nrows = min(nrows, *rows_dev);
  if (row >= nrows) return;
  const InT* xr = x + (size_t)row * cols;
  const int nblk = cols / 32;
  uint8_t* cr = codes + (size_t)row * cols;
  uint8_t* sr = scales + (size_t)row * nblk;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    float v[32];
    load_block<InT>(xr + 32 * b, 32, v);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) am = fmaxf(am, fabsf(v[i]));
    const int E = mx_exponent(am);
    const float step = pow2f(-E);   // -E in [-119, 127]
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      w[j] = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) w[j] |= e4m3_encode(__fmul_rn(v[4 * j + i], step)) << (8 * i);
    }
    uint4* dst = reinterpret_cast<uint4*>(cr + 32 * b);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    sr[b] = (uint8_t)(E + 127);
  }
}

int launch_quant(int fmt, int dtype, const void* x, int rows, const int* rows_dev, int cols,
                 uint8_t* codes, uint8_t* scales, float* gs, hipStream_t stream) {
  if (rows <= 0) return 0;
  const dim3 grid(rows), block(256);
  if (fmt == 1) {
    if (dtype == 0)
      hipLaunchKernelGGL(k_quant_nvfp4<uint16_t>, grid, block, 0, stream,
                         (const uint16_t*)x, rows, rows_dev, cols, codes, scales, gs);
    else
      hipLaunchKernelGGL(k_quant_nvfp4<float>, grid, block, 0, stream,
                         (const float*)x, rows, rows_dev, cols, codes, scales, gs);
  } else {
    if (dtype == 0)
      hipLaunchKernelGGL(k_quant_mxfp8<uint16_t>, grid, block, 0, stream,
                         (const uint16_t*)x, rows, rows_dev, cols, codes, scales);
    else
      hipLaunchKernelGGL(k_quant_mxfp8<float>, grid, block, 0, stream,
                         (const float*)x, rows, rows_dev, cols, codes, scales);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
