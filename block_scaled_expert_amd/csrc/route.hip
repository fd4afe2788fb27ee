// Router: z = x W_r^T on bf16 MFMA with fp32 accumulation, then per token
// sigmoid, additive selection bias and top-k with gate weights (SGLang blog
// "SGLang and Miles Add Day-0 Support for Inkling 2 Small", "Performance":
// the router's sigmoid, bias and top-k are one fused step; Miles docs
// section 1: sigmoid routing, 384 experts, top-8).
//
// Logits: a workgroup of 4 waves owns a (16*MS tokens) x (16*NS experts)
// tile; the waves split K four ways and their partial tiles are summed in a
// fixed order through LDS.  MFMA 16x16x32 bf16: lane l holds row l%16 and
// k-group l/16 of 8 elements; each lane loads 16 consecutive bf16 (32 bytes)
// and feeds them to two MFMAs, the B operand using the same k mapping.
#include "moe_common.h"
#include "launch.h"

namespace moe {

template <int MS, int NS>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x, int T, int H,
                                                       const uint16_t* __restrict__ wr, int E,
                                                       float* __restrict__ z) {
  __shared__ float red[4][16 * MS][16 * NS + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16 * MS, e0 = blockIdx.y * 16 * NS;
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = H / 64;                        // 64 k per step (two MFMAs)
  const int s_begin = wave * nsteps / 4, s_end = (wave + 1) * nsteps / 4;

  v4f acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int j = 0; j < NS; j++) acc[i][j] = v4f{0, 0, 0, 0};

  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  for (int s = s_begin; s < s_end; s++) {
    const int k0 = s * 64 + 16 * g;
    uint4 a[MS][2], b[NS][2];
#pragma unroll
    for (int i = 0; i < MS; i++) {
      const int t = t0 + 16 * i + r;
      if (t < T) {
        const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * H + k0);
        a[i][0] = p[0];
        a[i][1] = p[1];
      } else {
        a[i][0] = zero4;
        a[i][1] = zero4;
      }
    }
#pragma unroll
    for (int j = 0; j < NS; j++) {
      const int e = e0 + 16 * j + r;
      if (e < E) {
        const uint4* p = reinterpret_cast<const uint4*>(wr + (size_t)e * H + k0);
        b[j][0] = p[0];
        b[j][1] = p[1];
      } else {
        b[j][0] = zero4;
        b[j][1] = zero4;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < MS; i++)
#pragma unroll
        for (int j = 0; j < NS; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, a[i][h]), __builtin_bit_cast(v8bf, b[j][h]), acc[i][j], 0, 0, 0);
  }
  // output layout: acc reg q of lane l is D[4*(l/16)+q][l%16]
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int j = 0; j < NS; j++)
#pragma unroll
      for (int q = 0; q < 4; q++) red[wave][16 * i + 4 * g + q][16 * j + r] = acc[i][j][q];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * MS * 16 * NS; idx += 256) {
    const int m = idx / (16 * NS), n = idx % (16 * NS);
    const float v = ((red[0][m][n] + red[1][m][n]) + red[2][m][n]) + red[3][m][n];
    const int t = t0 + m, e = e0 + n;
    if (t < T && e < E) z[(size_t)t * E + e] = v;
  }
}

// One wave per token.  E <= 1024 (16 scores per lane), k <= 32.
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ z, int T, int E,
                                                     const float* __restrict__ bias, int k,
                                                     int norm_topk, float routed_scale,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w,
                                                     uint8_t* __restrict__ near_tie) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  constexpr int kMaxPer = 16;
  float sc[kMaxPer], sel[kMaxPer];
  const float* zt = z + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < kMaxPer; i++) {
    const int e = lane + 64 * i;
    if (e < E) {
      sc[i] = 1.0f / (1.0f + expf(-zt[e]));
      sel[i] = sc[i] + bias[e];
    } else {
      sc[i] = 0.0f;
      sel[i] = -INFINITY;
    }
  }
  float chosen_s = 0.0f;   // lane j < k keeps the score of the j-th choice
  int chosen_id = 0;
  float kth = 0.0f, next = -INFINITY;
  const int rounds = k < E ? k + 1 : k;
  for (int j = 0; j < rounds; j++) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPer; i++) {
      const int e = lane + 64 * i;
      if (e < E && (sel[i] > bv || (sel[i] == bv && e < bi))) {
        bv = sel[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == k) {
      next = bv;
      break;
    }
    if (j == k - 1) kth = bv;
    const int owner = bi & 63, slot = bi >> 6;
    float s_of = 0.0f;
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < kMaxPer; i++)
        if (i == slot) {
          s_of = sc[i];
          sel[i] = -INFINITY;
        }
    }
    s_of = __shfl(s_of, owner, kWave);
    if (lane == j) {
      chosen_s = s_of;
      chosen_id = bi;
    }
  }
  // gate weights: sum in j order
  float tot = 0.0f;
  for (int j = 0; j < k; j++) tot += __shfl(chosen_s, j, kWave);
  if (lane < k) {
    float wj = norm_topk ? chosen_s / tot : chosen_s;
    ids[(size_t)t * k + lane] = chosen_id;
    w[(size_t)t * k + lane] = wj * routed_scale;
  }
  if (lane == 0 && near_tie != nullptr) near_tie[t] = (k < E && (kth - next) < 1e-6f) ? 1 : 0;
}

int launch_router(const uint16_t* x, int T, int H, const uint16_t* wr, const float* bias, int E,
                  int k, int norm_topk, float routed_scale, float* z, int32_t* ids, float* w,
                  uint8_t* near_tie, hipStream_t stream) {
  if (T <= 0) return 0;
  if (T >= 2048) {
    const dim3 grid(ceil_div(T, 64), ceil_div(E, 64));
    hipLaunchKernelGGL((k_router_logits<4, 4>), grid, dim3(256), 0, stream, x, T, H, wr, E, z);
  } else {
    const dim3 grid(ceil_div(T, 16), ceil_div(E, 16));
    hipLaunchKernelGGL((k_router_logits<1, 1>), grid, dim3(256), 0, stream, x, T, H, wr, E, z);
  }
  hipLaunchKernelGGL(k_router_topk, dim3(ceil_div(T, 4)), dim3(256), 0, stream, z, T, E, bias, k,
                     norm_topk, routed_scale, ids, w, near_tie);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
