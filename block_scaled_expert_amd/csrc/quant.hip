// Activation quantization kernels: one workgroup of 256 threads per row (the
// row bodies and their format sources are in quant_row.h), and the two-pass
// maximum for an NVFP4 scale shared by a whole tensor.
// HBM-bound: every input byte is read once from HBM (the NVFP4 second pass
// hits the cache) and every output byte written once.
#include "quant_row.h"
#include "launch.h"

namespace moe {

// rows_dev (nullable): device row count that further limits rows.
template <typename InT, int MODE>
__global__ __launch_bounds__(256) void k_quant_nvfp4(const InT* __restrict__ x, int rows,
                                                     const int* __restrict__ rows_dev, int cols,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     float* __restrict__ gs_out, const float* __restrict__ gs_in,
                                                     float gs_val) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  int nrows = rows;
  if (rows_dev != nullptr) nrows = min(nrows, *rows_dev);
  if (row >= nrows) return;
  quant_row_nvfp4<InT, MODE>(x + (size_t)row * cols, cols, threadIdx.x, red, true, codes + (size_t)row * (cols / 2),
                             scales + (size_t)row * (cols / 16), gs_out + row, gs_in, gs_val);
}

template <typename InT>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const InT* __restrict__ x, int rows,
                                                     const int* __restrict__ rows_dev, int cols,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int row = blockIdx.x;
  int nrows = rows;
  if (rows_dev != nullptr) nrows = min(nrows, *rows_dev);
  if (row >= nrows) return;
  quant_row_mxfp8<InT>(x + (size_t)row * cols, cols, threadIdx.x, true, codes + (size_t)row * cols,
                       scales + (size_t)row * (cols / 32));
}

// Maximum magnitude of a [rows][cols] tensor, first pass: workgroup g of G
// takes rows [g n / G, (g+1) n / G) (n = rows, limited by *rows_dev) and
// writes their maximum to partial[g].  Max is order-independent, so the
// result does not depend on scheduling.
template <typename InT>
__global__ __launch_bounds__(256) void k_act_amax(const InT* __restrict__ x, int rows, const int* __restrict__ rows_dev,
                                                  int cols, float* __restrict__ partial) {
  __shared__ float red[4];
  int n = rows;
  if (rows_dev != nullptr) n = min(n, *rows_dev);
  const int G = gridDim.x, g = blockIdx.x, t = threadIdx.x;
  const long r0 = (long)g * n / G, r1 = (long)(g + 1) * n / G;
  const int nblk = cols / 16;
  float A = 0.0f;
  for (long r = r0; r < r1; r++) {
    const InT* xr = x + r * cols;
    for (int b = t; b < nblk; b += 256) {
      float v[16];
      load_block<InT>(xr + 16 * b, 16, v);
#pragma unroll
      for (int i = 0; i < 16; i++) A = fmaxf(A, fabsf(v[i]));
    }
  }
  A = group_max(A, red, t);
  if (t == 0) partial[g] = A;
}

// Second pass (one workgroup): the tensor's NVFP4 scale from the G partial
// maxima, to *gs.
__global__ __launch_bounds__(256) void k_act_gs_finish(const float* __restrict__ partial, int G,
                                                       float* __restrict__ gs) {
  __shared__ float red[4];
  float A = 0.0f;
  for (int i = threadIdx.x; i < G; i += 256) A = fmaxf(A, partial[i]);
  A = group_max(A, red, threadIdx.x);
  if (threadIdx.x == 0) *gs = nvfp4_gs(A);
}

int launch_act_gs_tensor(int dtype, const void* x, int rows, const int* rows_dev, int cols, float* scratch,
                         hipStream_t stream) {
  if (rows <= 0) return 0;
  const int G = rows < kActGsPartials ? rows : kActGsPartials;
  if (dtype == 0)
    hipLaunchKernelGGL(k_act_amax<uint16_t>, dim3(G), dim3(256), 0, stream, (const uint16_t*)x, rows, rows_dev, cols,
                       scratch + 1);
  else
    hipLaunchKernelGGL(k_act_amax<float>, dim3(G), dim3(256), 0, stream, (const float*)x, rows, rows_dev, cols,
                       scratch + 1);
  hipLaunchKernelGGL(k_act_gs_finish, dim3(1), dim3(256), 0, stream, scratch + 1, G, scratch);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quant(int fmt, int dtype, const void* x, int rows, const int* rows_dev, int cols,
                 uint8_t* codes, uint8_t* scales, float* gs, hipStream_t stream, const ActGs& ag) {
  if (rows <= 0) return 0;
  const dim3 grid(rows), block(256);
  if (fmt == 1) {
#define MOE_QNV(T, M)                                                                                            \
  hipLaunchKernelGGL((k_quant_nvfp4<T, M>), grid, block, 0, stream, (const T*)x, rows, rows_dev, cols, codes, \
                     scales, gs, ag.gs_dev, ag.gs_val)
#define MOE_QNV_T(T)                                 \
  do {                                               \
    if (ag.mode == GS_TENSOR) MOE_QNV(T, GS_TENSOR); \
    else if (ag.mode == GS_STATIC) MOE_QNV(T, GS_STATIC); \
    else MOE_QNV(T, GS_ROW);                         \
  } while (0)
    if (dtype == 0) MOE_QNV_T(uint16_t);
    else MOE_QNV_T(float);
#undef MOE_QNV_T
#undef MOE_QNV
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
