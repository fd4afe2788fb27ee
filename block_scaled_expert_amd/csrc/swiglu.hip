// The expert epilogue's capped SwiGLU as an elementwise kernel
// (moe_cap_swiglu): the same device function the gate/up GEMM epilogues
// call, so a caller can measure its error on chosen inputs.  Cap forms:
// SGLang cookbook "Inkling-2-Small" section 2 ("capped" SwiGLU), Miles docs
// "inkling-2-small" section 1 ("soft-capped").
#include "moe_common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void k_cap_swiglu(int form, float cap, float inv_c, const float* __restrict__ g,
                                                    const float* __restrict__ u, long n, float* __restrict__ h) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    h[i] = cap_swiglu(g[i], u[i], form, cap, inv_c);
}

int launch_cap_swiglu(int form, float cap, const float* g, const float* u, long n, float* h, hipStream_t stream) {
  if (n <= 0) return 0;
  const long blocks = (n + 255) / 256;
  const dim3 grid((unsigned)(blocks < 4096 ? blocks : 4096));
  hipLaunchKernelGGL(k_cap_swiglu, grid, dim3(256), 0, stream, form, cap, 1.0f / cap, g, u, n, h);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
