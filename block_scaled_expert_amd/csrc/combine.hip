// The combine stage as a kernel of its own: one workgroup per (token, 1024
// columns); the per-column body is in combine.h.
#include "combine.h"
#include "launch.h"

namespace moe {

template <bool NT>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int k, int H,
                                                 uint16_t* __restrict__ out) {
  const int c = blockIdx.y * 256 + threadIdx.x;     // float4 column
  if (c < H / 4) combine_col4<NT>(y, pos, w, k, H, out, blockIdx.x, c);
}

int launch_combine(const float* y, const int32_t* pos, const float* w, int T, int k, int H, bool nt,
                   uint16_t* out, hipStream_t stream) {
  if (T <= 0) return 0;
  const dim3 grid(T, ceil_div(H / 4, 256));
  if (nt) hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, stream, y, pos, w, k, H, out);
  else hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, stream, y, pos, w, k, H, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
