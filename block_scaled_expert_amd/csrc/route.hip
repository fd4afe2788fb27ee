// Router: z = x W_r^T on bf16 MFMA with fp32 accumulation, then per token
// sigmoid, additive selection bias and top-k with gate weights (SGLang blog
// "SGLang and Miles Add Day-0 Support for Inkling 2 Small", "Performance":
// the router's sigmoid, bias and top-k are one fused step; Miles docs
// section 1: sigmoid routing, 384 experts, top-8).
//
// Logits are computed as S partial sums over slices of K (S = 1..6) written
// to S planes; the top-k kernel adds them in slice order, so the result does
// not depend on scheduling.  MFMA 16x16x32 bf16: lane l holds row l%16 and
// k-group l/16 of 8 elements; each lane feeds 16 consecutive bf16 (32 bytes)
// to two MFMAs, the B operand using the same k mapping.
#include "moe_common.h"
#include "launch.h"

#include <algorithm>

namespace moe {

constexpr int kMaxSplits = 6;   // largest router_splits() value

// Small batches: the K range is also split over the grid's y dimension, so
// that the 3.5 MB router weight is streamed by many CUs at once.  Workgroup
// (expert tile x, split y, token group z) of 4 waves owns 16 experts x
// 16*MT tokens; each wave issues all loads of its k steps before its MFMAs.
// The partial sums zpart[y][t][e] are added in split order by the top-k
// kernel, so the result does not depend on scheduling.
template <int MT>
__global__ __launch_bounds__(256) void k_router_logits_split(const uint16_t* __restrict__ x, int T, int H,
                                                             const uint16_t* __restrict__ wr, int E, int S,
                                                             float* __restrict__ zpart) {
  constexpr int U = 3;                                // k steps per batch of loads
  __shared__ float red[4][16 * MT][17];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16, split = blockIdx.y, t0 = blockIdx.z * 16 * MT;
  const int nsteps = H / 64;
  const int s_lo = split * nsteps / S, s_hi = (split + 1) * nsteps / S;
  const int w_lo = s_lo + wave * (s_hi - s_lo) / 4, w_hi = s_lo + (wave + 1) * (s_hi - s_lo) / 4;

  // rows past E or T read a valid row; their sums are never stored
  const uint16_t* wrow = wr + (size_t)min(e0 + r, E - 1) * H + 16 * g;
  const uint16_t* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; i++) xrow[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * H + 16 * g;

  v4f acc[MT];
#pragma unroll
  for (int i = 0; i < MT; i++) acc[i] = v4f{0, 0, 0, 0};
  const v4u zero = v4u{0, 0, 0, 0};
  for (int s0 = w_lo; s0 < w_hi; s0 += U) {
    v4u b[U][2], a[U][MT][2];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int k0 = min(s0 + u, w_hi - 1) * 64;
      b[u][0] = *reinterpret_cast<const v4u*>(wrow + k0);
      b[u][1] = *reinterpret_cast<const v4u*>(wrow + k0 + 8);
#pragma unroll
      for (int i = 0; i < MT; i++) {
        a[u][i][0] = *reinterpret_cast<const v4u*>(xrow[i] + k0);
        a[u][i][1] = *reinterpret_cast<const v4u*>(xrow[i] + k0 + 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const bool live = s0 + u < w_hi;               // a repeated step adds zero
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const v4u bv = live ? b[u][h] : zero;
#pragma unroll
        for (int i = 0; i < MT; i++)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u][i][h]),
                                                           __builtin_bit_cast(v8bf, bv), acc[i], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; i++)
#pragma unroll
    for (int q = 0; q < 4; q++) red[wave][16 * i + 4 * g + q][r] = acc[i][q];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * MT * 16; idx += 256) {
    const int m = idx >> 4, n = idx & 15;
    const float v = ((red[0][m][n] + red[1][m][n]) + red[2][m][n]) + red[3][m][n];
    const int t = t0 + m, e = e0 + n;
    if (t < T && e < E) zpart[((size_t)split * T + t) * E + e] = v;
  }
}

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

// Selection keys: the fp32 selection score mapped to an unsigned integer of
// the same order, above the complement of the expert id, so that the larger
// key is the larger score and, between equal scores, the lower expert.
// Key 0 is below every real key.
__device__ inline uint64_t sel_key(float v, int e) {
  const uint32_t b = f_bits(v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ inline float key_score(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return bits_f((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ inline int key_expert(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ inline uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Maximum over the wavefront: inside each row of 16 lanes with DPP (swap
// neighbours, swap pairs, mirror the half rows, mirror the row), then over the
// four rows.  The result is wave-uniform.
__device__ inline uint64_t wave_max_key(uint64_t k) {
  uint64_t o;
  o = dpp_u64<0xB1>(k);  k = o > k ? o : k;    // quad_perm [1,0,3,2]
  o = dpp_u64<0x4E>(k);  k = o > k ? o : k;    // quad_perm [2,3,0,1]
  o = dpp_u64<0x141>(k); k = o > k ? o : k;    // row_half_mirror
  o = dpp_u64<0x140>(k); k = o > k ? o : k;    // row_mirror
  const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
  const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// One wave per token; lane l holds experts l + 64 i.  Logits are the sum of
// S split partials (S = 1: the plain logits), added in split order.  k + 1
// rounds of a wavefront arg-max give the top-k and the (k+1)-th score for
// the near-tie flag.  E <= 64 * NPER, k <= 32.
template <int NPER>
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ zpart, int S, int T, int E,
                                                     const float* __restrict__ bias, int k,
                                                     int norm_topk, float routed_scale,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w,
                                                     uint8_t* __restrict__ near_tie) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float sc[NPER];
  uint64_t key[NPER];
  // every load in one batch (clamped addresses, no branches); splits past S
  // add +0, which leaves the sum unchanged
  const size_t split_stride = (size_t)T * E;
  float zz[NPER][kMaxSplits], bb[NPER];
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int ec = min(lane + 64 * i, E - 1);
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; sp++) zz[i][sp] = zpart[min(sp, S - 1) * split_stride + (size_t)t * E + ec];
    bb[i] = bias[ec];
  }
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int e = lane + 64 * i;
    float z = zz[i][0];
#pragma unroll
    for (int sp = 1; sp < kMaxSplits; sp++) z += sp < S ? zz[i][sp] : 0.0f;
    sc[i] = 1.0f / (1.0f + expf(-z));
    key[i] = e < E ? sel_key(sc[i] + bb[i], e) : 0ull;
  }
  float chosen_s = 0.0f;   // lane j < k keeps the score of the j-th choice
  int chosen_id = 0;
  float tot = 0.0f, kth = 0.0f, next = -INFINITY;
  const int rounds = k < E ? k + 1 : k;
  for (int j = 0; j < rounds; j++) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < NPER; i++) m = key[i] > m ? key[i] : m;
    const uint64_t best = wave_max_key(m);
    if (j == k) {
      next = key_score(best);
      break;
    }
    const int be = key_expert(best);
    if (j == k - 1) kth = key_score(best);
    const int owner = be & 63, slot = be >> 6;
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; i++) {
      v = i == slot ? sc[i] : v;
      if (lane == owner && i == slot) key[i] = 0ull;
    }
    const float s_of = bits_f(__builtin_amdgcn_readlane((int)f_bits(v), owner));
    tot += s_of;                                      // gate-weight sum in j order
    if (lane == j) {
      chosen_s = s_of;
      chosen_id = be;
    }
  }
  if (lane < k) {
    const float wj = norm_topk ? chosen_s / tot : chosen_s;
    ids[(size_t)t * k + lane] = chosen_id;
    w[(size_t)t * k + lane] = wj * routed_scale;
  }
  if (lane == 0 && near_tie != nullptr) near_tie[t] = (k < E && (kth - next) < 1e-6f) ? 1 : 0;
}

// K splits: small batches (split-K GEMV, 6 / 4 / 2 planes); larger ones
// (128 x 128 tiles, two workgroups per CU) take as many splits as keep the
// grid within 512 workgroups, at most 6.
int router_splits(int T, int E) {
  if (T <= 256) return T <= 64 ? 6 : T <= 128 ? 4 : 2;
  const int tiles = ceil_div(T, 128) * ceil_div(E, 128);
  return std::min(kMaxSplits, std::max(1, 512 / tiles));   // one round of 512 workgroup slots
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
