// Device bodies of the router kernels, shared by the router launches
// (route.hip) and the small-batch route + quantize + dispatch launch
// (route_prep.hip).  Router: z = x W_r^T on bf16 MFMA with fp32
// accumulation, then per token sigmoid, additive selection bias and top-k
// with gate weights (SGLang blog "SGLang and Miles Add Day-0 Support for
// Inkling 2 Small", "Performance": sigmoid, bias and top-k fused; Miles docs
// section 1: sigmoid routing, 384 experts, top-8).
//
// Logits are computed as S partial sums over slices of K written to S
// planes; the top-k adds them in slice order, so the result does not depend
// on scheduling.  MFMA 16x16x32 bf16: lane l holds row l%16 and k-group l/16
// of 8 elements; each lane feeds 16 consecutive bf16 (32 bytes) to two
// MFMAs, the B operand using the same k mapping.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kMaxSplits = 6;   // largest router_splits() value

// Small batches: the K range is also split over the grid's y dimension, so
// that the 3.5 MB router weight is streamed by many CUs at once.  Workgroup
// (expert tile x, split y, token group z) of 4 waves owns 16 experts x
// 16*MT tokens; each wave issues all loads of its k steps before its MFMAs.
// The partial sums zpart[y][t][e] are added in split order by the top-k
// kernel, so the result does not depend on scheduling.
template <int MT>
struct SplitLds {
  float red[4][16 * MT][17];
};

// One workgroup's tile of the split-K GEMV: experts 16 ex .., K slice
// `split` of S, tokens 16 MT tg ..; every thread of the 256-thread
// workgroup calls it (tid: its index).  COH: the partial sums are stored at
// device scope (written through, for readers in the same launch).
template <int MT, bool COH = false>
__device__ __forceinline__ void router_logits_split_tile(const uint16_t* __restrict__ x, int T, int H,
                                                         const uint16_t* __restrict__ wr, int E, int S,
                                                         float* __restrict__ zpart, int ex, int split, int tg,
                                                         SplitLds<MT>& sm, int tid) {
  constexpr int U = 3;                                // k steps per batch of loads
  auto& red = sm.red;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = ex * 16, t0 = tg * 16 * MT;
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
  for (int idx = tid; idx < 16 * MT * 16; idx += 256) {
    const int m = idx >> 4, n = idx & 15;
    const float v = ((red[0][m][n] + red[1][m][n]) + red[2][m][n]) + red[3][m][n];
    const int t = t0 + m, e = e0 + n;
    if (t < T && e < E) {
      float* p = zpart + ((size_t)split * T + t) * E + e;
      if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *p = v;
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
// One wave's token t (t < T).  COH: ids and weights stored at device scope.
template <int NPER, bool COH = false>
__device__ __forceinline__ void router_topk_token(const float* __restrict__ zpart, int S, int T, int E,
                                                  const float* __restrict__ bias, int k, int norm_topk,
                                                  float routed_scale, int32_t* __restrict__ ids,
                                                  float* __restrict__ w, uint8_t* __restrict__ near_tie, int t,
                                                  int lane) {
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
    if constexpr (COH) {
      __hip_atomic_store(ids + (size_t)t * k + lane, chosen_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(w + (size_t)t * k + lane, wj * routed_scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      ids[(size_t)t * k + lane] = chosen_id;
      w[(size_t)t * k + lane] = wj * routed_scale;
    }
  }
  if (lane == 0 && near_tie != nullptr) near_tie[t] = (k < E && (kth - next) < 1e-6f) ? 1 : 0;
}



}  // namespace moe
