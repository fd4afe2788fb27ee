// Deterministic weighted combine: out[t] = bf16_rne(sum_j w[t][j] * y[t, j])
// summed in fixed j order over the pairs whose expert is local (the
// "combine" stage of the SGLang cookbook's MegaMoE description, section 2).
// y rows are in expert-sorted order; pair_pos maps pair t*k + j to its row
// (-1: expert not local).  One workgroup per (token, 1024 columns), fp32
// accumulation, no atomics.  HBM-bound: reads k rows of fp32 y, writes one
// bf16 row.  y larger than the last-level cache is read with the
// non-temporal hint (NT).
#include "moe_common.h"
#include "launch.h"

namespace moe {

template <bool NT>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int k, int H,
                                                 uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int32_t* pt = pos + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  const int c = blockIdx.y * 256 + threadIdx.x;     // float4 column
  if (c < H / 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
      const int p = pt[j];
      if (p < 0) continue;
      const float wj = wt[j];
      const v4f* yp = reinterpret_cast<const v4f*>(y + (size_t)p * H) + c;
      const v4f v = NT ? __builtin_nontemporal_load(yp) : *yp;
      acc.x += wj * v.x;
      acc.y += wj * v.y;
      acc.z += wj * v.z;
      acc.w += wj * v.w;
    }
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(out + (size_t)t * H)[c] = make_uint2(lo, hi);
  }
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
