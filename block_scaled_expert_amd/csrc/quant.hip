// Per-row activation quantization kernels: one workgroup of 256 threads per
// row (the row bodies and their format sources are in quant_row.h).
// HBM-bound: every input byte is read once from HBM (the NVFP4 second pass
// hits the cache) and every output byte written once.
#include "quant_row.h"
#include "launch.h"

namespace moe {

// rows_dev (nullable): device row count that further limits rows.
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
  quant_row_nvfp4<InT>(x + (size_t)row * cols, cols, threadIdx.x, red, true, codes + (size_t)row * (cols / 2),
                       scales + (size_t)row * (cols / 16), gs_out + row);
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
