// Deterministic weighted combine: out[t] = bf16_rne(sum_j w[t][j] * y[t, j])
// summed in fixed j order over the pairs whose expert is local (the
// "combine" stage of the SGLang cookbook's MegaMoE description, section 2).
// y rows are in expert-sorted order; pair_pos maps pair t*k + j to its row
// (-1: expert not local).  fp32 accumulation, no atomics.  HBM-bound: reads
// k rows of fp32 y, writes one bf16 row.  y larger than the last-level cache
// is read with the non-temporal hint (NT).
#pragma once

#include "moe_common.h"

namespace moe {

// Token t, float4 column c (c < H / 4: one thread each).
template <bool NT>
__device__ inline void combine_col4(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                    const float* __restrict__ w, int k, int H, uint16_t* __restrict__ out, int t,
                                    int c) {
  const int32_t* pt = pos + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
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

}  // namespace moe
