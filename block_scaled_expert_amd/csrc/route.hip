// Router launches: the logits (split-K GEMV planes for small batches,
// LDS-tiled 128 x 128 tiles above 256 tokens), then sigmoid + bias + top-k
// (one wave per token).  Bodies and sources in route_body.h.
#include "route_body.h"
#include "launch.h"

#include <algorithm>

namespace moe {

// Larger batches: a workgroup of 8 waves (2 x 4) computes a 128-token x
// 128-expert tile over one K slice (grid z = split).  Each 64-wide k step of
// both operands is staged in LDS in MFMA lane order (chunk q of 16 bytes at
// byte 16 q: row tile q/128, k half (q/64)%2, lane q%64), so every wavefront
// store and load is 1 KB contiguous; the steps after the current one are
// fetched into registers while it is multiplied.  Each wave owns 64 tokens x
// 32 experts over the whole slice (half the accumulators of a 2 x 2
// arrangement), so the kernel fits 128 registers and two workgroups share a
// CU (4 waves per SIMD); each wave writes its partial plane directly.  Every
// output's k order is the same as in one wave: step by step, both halves.
__global__ __launch_bounds__(512, 4) void k_router_logits_tiled(const uint16_t* __restrict__ x, int T, int H,
                                                                const uint16_t* __restrict__ wr, int E, int S,
                                                                float* __restrict__ zpart) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][16384];   // [buffer][A, B][8 tiles x 2 halves x 64 lanes x 16 B]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * 128, e0 = blockIdx.y * 128, split = blockIdx.z;
  const int nsteps = H / 64;
  const int s_lo = split * nsteps / S, s_hi = (split + 1) * nsteps / S;

  // staging: thread takes chunks q = tid + 512 u (u < 2) of each operand;
  // rows past T / E read a valid row (their sums are never stored)
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int q = tid + 512 * u, f = q >> 7, hh = (q >> 6) & 1, l = q & 63;
    const int koff = 32 * hh + 8 * (l >> 4);
    ap[u] = x + (size_t)min(t0 + 16 * f + (l & 15), T - 1) * H + koff;
    bp[u] = wr + (size_t)min(e0 + 16 * f + (l & 15), E - 1) * H + koff;
  }
  // two register stages: a step's global loads are issued two steps before
  // its MFMAs (one step before its LDS store)
  v4u ra[2][2], rb[2][2];
  auto gload = [&](int st, v4u (&sa)[2], v4u (&sb)[2]) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      sa[u] = *reinterpret_cast<const v4u*>(ap[u] + st * 64);
      sb[u] = *reinterpret_cast<const v4u*>(bp[u] + st * 64);
    }
  };
  auto lstore = [&](int buf, const v4u (&sa)[2], const v4u (&sb)[2]) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      *reinterpret_cast<v4u*>(&lds[buf][0][16 * (tid + 512 * u)]) = sa[u];
      *reinterpret_cast<v4u*>(&lds[buf][1][16 * (tid + 512 * u)]) = sb[u];
    }
  };

  v4f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++) acc[i][0] = acc[i][1] = v4f{0, 0, 0, 0};
  auto mma = [&](int buf) {
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      v4u av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; i++)
        av[i] = *reinterpret_cast<const v4u*>(&lds[buf][0][16 * ((4 * wm + i) * 128 + hh * 64 + lane)]);
#pragma unroll
      for (int j = 0; j < 2; j++)
        bv[j] = *reinterpret_cast<const v4u*>(&lds[buf][1][16 * ((2 * wn + j) * 128 + hh * 64 + lane)]);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[i]),
                                                              __builtin_bit_cast(v8bf, bv[j]), acc[i][j], 0, 0, 0);
    }
  };

  // Steps s_lo + 2n use LDS buffer 0, s_lo + 2n + 1 buffer 1; a buffer is
  // rewritten only after the barrier that follows its last read.  Loads past
  // the slice re-read its last step; a missing odd last step is skipped.
  if (s_hi > s_lo) {
    gload(s_lo, ra[0], rb[0]);
    lstore(0, ra[0], rb[0]);
    gload(min(s_lo + 1, s_hi - 1), ra[0], rb[0]);
    gload(min(s_lo + 2, s_hi - 1), ra[1], rb[1]);
    __syncthreads();
    for (int st = s_lo; st < s_hi; st += 2) {
      mma(0);                                           // step st
      lstore(1, ra[0], rb[0]);                          // step st + 1
      gload(min(st + 3, s_hi - 1), ra[0], rb[0]);
      __syncthreads();
      if (st + 1 < s_hi) mma(1);                        // step st + 1
      lstore(0, ra[1], rb[1]);                          // step st + 2
      gload(min(st + 4, s_hi - 1), ra[1], rb[1]);
      __syncthreads();
    }
  }
  // acc reg q of lane l in tile (i, j): token row 16 i + 4 (l/16) + q of the
  // wave's 64, expert column 16 j + l%16 of its 32
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int t = t0 + 64 * wm + 16 * i + 4 * g + q;
      if (t >= T) continue;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int e = e0 + 32 * wn + 16 * j + r;
        if (e < E) zpart[((size_t)split * T + t) * E + e] = acc[i][j][q];
      }
    }
}

// Small batches: workgroup (16 experts x, K slice y, 16 MT tokens z) of 4
// waves; the partial planes are added in slice order by the top-k.
template <int MT>
__global__ __launch_bounds__(256) void k_router_logits_split(const uint16_t* __restrict__ x, int T, int H,
                                                             const uint16_t* __restrict__ wr, int E, int S,
                                                             float* __restrict__ zpart) {
  __shared__ SplitLds<MT> sm;
  router_logits_split_tile<MT>(x, T, H, wr, E, S, zpart, blockIdx.x, blockIdx.y, blockIdx.z, sm, threadIdx.x);
}

// One wave per token.
template <int NPER>
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ zpart, int S, int T, int E,
                                                     const float* __restrict__ bias, int k,
                                                     int norm_topk, float routed_scale,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w,
                                                     uint8_t* __restrict__ near_tie) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  router_topk_token<NPER>(zpart, S, T, E, bias, k, norm_topk, routed_scale, ids, w, near_tie, t,
                          threadIdx.x & 63);
}

// K splits: small batches (split-K GEMV, 6 / 4 / 2 planes); larger ones
// (128 x 128 tiles) take as many splits as keep the grid within 256
// workgroups, between 2 and 6.  Measured on MI355X (router logits + top-k,
// 384 experts, by splits 1..6): the time steps up wherever the grid passes
// 256 workgroups, and 2 slices beat 1 when the tiles alone exceed 256
// (2048 tokens: 41.5 us at 6 splits, 31.2 at 5; 4096: 52.7 at 5, 51.3 at
// 2; 16384: 179.9 at 1, 144.9 at 2).
int router_splits(int T, int E) {
  if (T <= 256) return T <= 64 ? 6 : T <= 128 ? 4 : 2;
  const int tiles = ceil_div(T, 128) * ceil_div(E, 128);
  return std::min(kMaxSplits, std::max(2, 256 / tiles));
}

size_t router_z_rows(int max_tokens) { return (size_t)kMaxSplits * (size_t)std::max(max_tokens, 0); }

int launch_router(const uint16_t* x, int T, int H, const uint16_t* wr, const float* bias, int E,
                  int k, int norm_topk, float routed_scale, float* z, int32_t* ids, float* w,
                  uint8_t* near_tie, hipStream_t stream) {
  if (T <= 0) return 0;
  const int S = router_splits(T, E);
  if (T <= 256) {
    const int mt = T <= 16 ? 1 : T <= 32 ? 2 : 4;
    const dim3 grid(ceil_div(E, 16), S, ceil_div(T, 16 * mt));
    if (mt == 1) hipLaunchKernelGGL((k_router_logits_split<1>), grid, dim3(256), 0, stream, x, T, H, wr, E, S, z);
    else if (mt == 2) hipLaunchKernelGGL((k_router_logits_split<2>), grid, dim3(256), 0, stream, x, T, H, wr, E, S, z);
    else hipLaunchKernelGGL((k_router_logits_split<4>), grid, dim3(256), 0, stream, x, T, H, wr, E, S, z);
  } else {
    const dim3 grid(ceil_div(T, 128), ceil_div(E, 128), S);
    hipLaunchKernelGGL(k_router_logits_tiled, grid, dim3(512), 0, stream, x, T, H, wr, E, S, z);
  }
  const dim3 tg(ceil_div(T, 4));
#define MOE_TOPK(N) \
  hipLaunchKernelGGL(k_router_topk<N>, tg, dim3(256), 0, stream, z, S, T, E, bias, k, norm_topk, routed_scale, ids, w, near_tie)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
