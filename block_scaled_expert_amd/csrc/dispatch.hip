// Dispatch: a stable counting sort of the (token, slot) pair ids p = t*k + j
// by local expert id, plus the per-expert tile work list the grouped GEMMs
// walk.  This is the "dispatch" stage that precedes both expert GEMMs in the
// SGLang cookbook's MegaMoE description (section 2, "MegaMoE").
//
// Batches of more than 4096 pairs take four launches (smaller ones one; see
// k_disp_small), with no floating point and no order-deciding atomics:
//   count   one workgroup per chunk of pairs: LDS histogram -> counts[c][e]
//   scan    one workgroup per expert: exclusive scan of counts[*][e] over
//           chunks (chunk order = pair order) -> per-chunk bases, totals[e]
//   offsets one workgroup: exclusive scan of totals over experts; the GEMM
//           tile list (local expert, first row) with tile_m rows per tile
//   scatter one workgroup per chunk: each pair's rank among the earlier
//           pairs of its expert inside the chunk (ballots within a
//           wavefront, running counts across wavefronts) gives its sorted
//           position; integer atomics only accumulate counts.
#include "moe_common.h"
#include "launch.h"
#include "quant_row.h"
#include "route_body.h"

namespace moe {

constexpr int kSub = 256;   // pairs handled per pass of a 256-thread workgroup

int dispatch_chunk(int P) {
  // at most 1024 chunks so one 1024-thread workgroup can scan an expert
  const int c = ceil_div(P, 1024);
  return c <= kSub ? kSub : ceil_div(c, kSub) * kSub;
}

__global__ __launch_bounds__(256) void k_disp_count(const int32_t* __restrict__ ids, int P, int chunk,
                                                    int E_begin, int E_local, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E_local; e += 256) hist[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int end = min(P, (c + 1) * chunk);
  for (int p = c * chunk + threadIdx.x; p < end; p += 256) {
    const int e = ids[p] - E_begin;
    if (e >= 0 && e < E_local) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E_local; e += 256) counts[(size_t)c * E_local + e] = hist[e];
}

// grid = E_local, block = 1024; nchunks <= 1024.  counts[c][e] becomes the
// number of pairs of expert e in chunks before c.
__global__ __launch_bounds__(1024) void k_disp_scan(int32_t* __restrict__ counts, int nchunks, int E_local,
                                                    int32_t* __restrict__ totals) {
  __shared__ int32_t s[1024];
  const int e = blockIdx.x, i = threadIdx.x;
  const int v = i < nchunks ? counts[(size_t)i * E_local + e] : 0;
  s[i] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {        // Hillis-Steele inclusive scan
    const int add = i >= o ? s[i - o] : 0;
    __syncthreads();
    s[i] += add;
    __syncthreads();
  }
  if (i < nchunks) counts[(size_t)i * E_local + e] = s[i] - v;
  if (i == 1023) totals[e] = s[1023];
}

// One 1024-thread workgroup; E_local <= 1024.
__global__ __launch_bounds__(1024) void k_disp_offsets(const int32_t* __restrict__ totals, int E_local,
                                                       int tile_m, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ worklist,
                                                       int32_t* __restrict__ ntiles) {
  __shared__ int32_t s[1024], st[1024];
  const int i = threadIdx.x;
  const int n = i < E_local ? totals[i] : 0;
  const int nt = (n + tile_m - 1) / tile_m;
  s[i] = n;
  st[i] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = i >= o ? s[i - o] : 0;
    const int b = i >= o ? st[i - o] : 0;
    __syncthreads();
    s[i] += a;
    st[i] += b;
    __syncthreads();
  }
  if (i < E_local) offsets[i] = s[i] - n;
  if (i == 0) offsets[E_local] = s[1023];
  if (i == 1023 && ntiles != nullptr) ntiles[0] = st[1023];
  if (worklist != nullptr && i < E_local) {
    const int base = st[i] - nt;
    for (int j = 0; j < nt; j++) {
      worklist[2 * (base + j)] = i;
      worklist[2 * (base + j) + 1] = j * tile_m;
    }
  }
}

// Lanes of the calling wavefront whose value of v (11 bits) equals this
// lane's: one ballot per bit.
__device__ inline uint64_t same_value_lanes(uint32_t v) {
  uint64_t same = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; b++) {
    const uint64_t bal = __ballot((v >> b) & 1u);
    same &= ((v >> b) & 1u) ? bal : ~bal;
  }
  return same;
}

// One workgroup per chunk, passes of 256 pairs.  A pair's sorted position is
// its expert's offset + the pairs of that expert in earlier chunks (the
// scan) + those placed by earlier passes and wavefronts of this chunk (run[],
// advanced wavefront by wavefront) + its rank among the lanes of its
// wavefront with the same expert (ballots).
__global__ __launch_bounds__(256) void k_disp_scatter(const int32_t* __restrict__ ids, int P, int chunk,
                                                      int E_begin, int E_local,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ pos) {
  extern __shared__ int32_t run[];            // [E_local] pairs already placed in this chunk
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E_local; e += 256) run[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int begin = c * chunk, end = min(P, (c + 1) * chunk);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int p0 = begin; p0 < end; p0 += kSub) {
    const int p = p0 + tid;
    int e = -1;
    if (p < end) {
      e = ids[p] - E_begin;
      if (e < 0 || e >= E_local) e = -1;
    }
    if (p < end && e < 0 && pos != nullptr) pos[p] = -1;
    const uint64_t same = same_value_lanes((uint32_t)(e + 1));
    const int rank = __popcll(same & below);
    const int total = __popcll(same);
    const bool last = (same & ~below & ~(1ull << lane)) == 0ull;
    const int waves = min(kSub / 64, (end - p0 + 63) / 64);
    for (int w = 0; w < waves; w++) {
      if (wave == w && e >= 0) {
        const int base = run[e];               // read by every lane before the last lane writes
        const int q = offsets[e] + counts[(size_t)c * E_local + e] + base + rank;
        if (sorted != nullptr) sorted[q] = p;
        if (pos != nullptr) pos[p] = q;
        if (last) run[e] = base + total;
      }
      __syncthreads();
    }
  }
}

// Small batches (P <= kSmallP pairs): the whole dispatch in one 1024-thread
// workgroup -- LDS histogram, one scan over the experts (offsets and the tile
// list), then passes of 1024 pairs.  In a pass each wavefront finds, with
// ballots over the bits of the expert id, the lanes that share a lane's
// expert; a pair's rank is the number of such lanes below it plus the pairs
// of that expert placed before its wavefront, which the wavefronts add to a
// running per-expert count in wavefront order.
constexpr int kSmallP = kSmallDispatchPairs;

// Body of the small-batch dispatch for one workgroup of 1024 threads.
__device__ inline void disp_small_body(const int32_t* __restrict__ ids, int P, int E_begin, int E_local,
                                       int tile_m, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                       int32_t* __restrict__ pos, int32_t* __restrict__ worklist,
                                       int32_t* __restrict__ ntiles) {
  __shared__ int32_t cnt[1024], off[1024], toff[1024];
  const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
  cnt[i] = 0;
  __syncthreads();
  for (int p = i; p < P; p += 1024) {
    const int e = ids[p] - E_begin;
    if (e >= 0 && e < E_local) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int n = i < E_local ? cnt[i] : 0;
  const int nt = (n + tile_m - 1) / tile_m;
  off[i] = n;
  toff[i] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {        // inclusive scans of counts and tiles
    const int a = i >= o ? off[i - o] : 0;
    const int b = i >= o ? toff[i - o] : 0;
    __syncthreads();
    off[i] += a;
    toff[i] += b;
    __syncthreads();
  }
  const int excl = off[i] - n;
  if (i < E_local) offsets[i] = excl;
  if (i == 0) offsets[E_local] = off[1023];
  if (i == 1023 && ntiles != nullptr) ntiles[0] = toff[1023];
  if (worklist != nullptr && i < E_local) {
    const int base = toff[i] - nt;
    for (int j = 0; j < nt; j++) {
      worklist[2 * (base + j)] = i;
      worklist[2 * (base + j) + 1] = j * tile_m;
    }
  }
  __syncthreads();
  off[i] = excl;                               // exclusive offsets
  cnt[i] = 0;                                  // pairs placed so far, per expert
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int p0 = 0; p0 < P; p0 += 1024) {
    const int p = p0 + i;
    int e = -1;
    if (p < P) {
      e = ids[p] - E_begin;
      if (e < 0 || e >= E_local) e = -1;
    }
    if (p < P && e < 0 && pos != nullptr) pos[p] = -1;
    const uint64_t same = same_value_lanes((uint32_t)(e + 1));
    const int rank = __popcll(same & below);
    const int total = __popcll(same);
    const bool last = (same & ~below & ~(1ull << lane)) == 0ull;
    const int waves = min(16, (P - p0 + 63) / 64);   // wavefronts holding pairs
    for (int w = 0; w < waves; w++) {
      if (wave == w && e >= 0) {
        const int base = cnt[e];               // read by every lane before the last lane writes
        const int q = off[e] + base + rank;
        if (sorted != nullptr) sorted[q] = p;
        if (pos != nullptr) pos[p] = q;
        if (last) cnt[e] = base + total;
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(1024) void k_disp_small(const int32_t* __restrict__ ids, int P, int E_begin,
                                                     int E_local, int tile_m, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ worklist,
                                                     int32_t* __restrict__ ntiles) {
  disp_small_body(ids, P, E_begin, E_local, tile_m, offsets, sorted, pos, worklist, ntiles);
}

// The same dispatch by one 256-thread workgroup (the items of the
// small-batch route + prepare launch below are 256 threads): thread i holds
// experts 4i .. 4i+3 for the scans; pairs are placed in passes of 256.
struct Disp256Lds {
  int32_t cnt[1024], off[1024], part[256], tpart[256];
};
__device__ inline void disp_small_body256(const int32_t* __restrict__ ids, int P, int E_begin, int E_local,
                                          int tile_m, int32_t* __restrict__ offsets,
                                          int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
                                          int32_t* __restrict__ worklist, int32_t* __restrict__ ntiles,
                                          Disp256Lds& sm) {
  const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
  for (int e = i; e < 1024; e += 256) sm.cnt[e] = 0;
  __syncthreads();
  for (int p = i; p < P; p += 256) {
    const int e = ids[p] - E_begin;
    if (e >= 0 && e < E_local) atomicAdd(&sm.cnt[e], 1);
  }
  __syncthreads();
  int n[4], nt[4], sn = 0, snt = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = 4 * i + j;
    n[j] = e < E_local ? sm.cnt[e] : 0;
    nt[j] = (n[j] + tile_m - 1) / tile_m;
    sn += n[j];
    snt += nt[j];
  }
  sm.part[i] = sn;
  sm.tpart[i] = snt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {          // inclusive scans of the per-thread totals
    const int a = i >= o ? sm.part[i - o] : 0;
    const int b = i >= o ? sm.tpart[i - o] : 0;
    __syncthreads();
    sm.part[i] += a;
    sm.tpart[i] += b;
    __syncthreads();
  }
  int base = sm.part[i] - sn, tbase = sm.tpart[i] - snt;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = 4 * i + j;
    if (e < E_local) {
      offsets[e] = base;
      if (worklist != nullptr)
        for (int jj = 0; jj < nt[j]; jj++) {
          worklist[2 * (tbase + jj)] = e;
          worklist[2 * (tbase + jj) + 1] = jj * tile_m;
        }
    }
    sm.off[e] = base;
    base += n[j];
    tbase += nt[j];
  }
  if (i == 0) offsets[E_local] = sm.part[255];
  if (i == 0 && ntiles != nullptr) ntiles[0] = sm.tpart[255];
  __syncthreads();
  for (int e = i; e < 1024; e += 256) sm.cnt[e] = 0;   // pairs placed so far, per expert
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int p0 = 0; p0 < P; p0 += 256) {
    const int p = p0 + i;
    int e = -1;
    if (p < P) {
      e = ids[p] - E_begin;
      if (e < 0 || e >= E_local) e = -1;
    }
    if (p < P && e < 0 && pos != nullptr) pos[p] = -1;
    const uint64_t same = same_value_lanes((uint32_t)(e + 1));
    const int rank = __popcll(same & below);
    const int total = __popcll(same);
    const bool last = (same & ~below & ~(1ull << lane)) == 0ull;
    const int waves = min(4, (P - p0 + 63) / 64);
    for (int w = 0; w < waves; w++) {
      if (wave == w && e >= 0) {
        const int b0 = sm.cnt[e];              // read by every lane before the last lane writes
        const int q = sm.off[e] + b0 + rank;
        if (sorted != nullptr) sorted[q] = p;
        if (pos != nullptr) pos[p] = q;
        if (last) sm.cnt[e] = b0 + total;
      }
      __syncthreads();
    }
  }
}

// Small batches (T <= 256 tokens, T k <= 4096 pairs): routing, the
// quantization of the token rows and the dispatch in ONE launch (the
// small-batch decode path, where the layer is bound by launches and their
// dependency waits: TokenSpeed blog, the paragraph after the "What's new"
// table; SGLang blog "Performance").  One 256-thread workgroup per item, in
// index order:
//   logits  (16 experts, K slice, 16 MT tokens)   the split-K GEMV tiles
//   quant   (token row)                            x in the layer's format
//   top-k   (4 tokens)                             after its token group's logits
//   dispatch                                       after every top-k item
// An item waits only for items of lower index, which the hardware has
// dispatched before it; at these sizes the whole grid is resident on the
// chip at once.  Completion is published per item as a 64-bit flag equal
// to this call's epoch (a per-call value from the host): flags left by
// earlier calls, or whatever the workspace held, never equal it, so no
// clearing launch is needed.  Results another item reads (partial logits,
// ids, weights) are stored at device scope and completed before the flag;
// a waiting item acquires after its flags.  Waits are bounded: one that
// runs out writes NaN gate weights for its tokens (their outputs become
// NaN) and goes on, so every wave reaches the end.
constexpr uint32_t kPrepSpin = 1u << 20;

// Every thread polls its share of the n flags; true if all were seen.
__device__ inline bool wait_epoch_flags(const uint64_t* f, int n, uint64_t epoch) {
  bool ok = true;
  for (int i = threadIdx.x; i < n; i += 256) {
    for (uint32_t it = 0;; it++) {
      if (__hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) break;
      if (it >= kPrepSpin) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  ok = __syncthreads_and(ok);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// Wait for this workgroup's stores, then publish the flag.
__device__ inline void publish_epoch(uint64_t* f, uint64_t epoch) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(f, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int GSM, int MT, int NPER>
__global__ __launch_bounds__(256) void k_route_prep(RoutePrepArgs a) {
  __shared__ union {
    SplitLds<MT> lg;
    Disp256Lds d;
    float red[4];
  } sm;
  const int tid = threadIdx.x;
  const int nex = (a.E + 15) / 16;
  const int ntg = (a.T + 16 * MT - 1) / (16 * MT);
  const int n_logits = nex * a.S * ntg, n_topk = (a.T + 3) / 4;
  int b = blockIdx.x;
  if (b < n_logits) {
    const int ex = b % nex, rest = b / nex, split = rest % a.S, tg = rest / a.S;
    router_logits_split_tile<MT, true>(a.x, a.T, a.H, a.wr, a.E, a.S, a.z, ex, split, tg, sm.lg, tid);
    publish_epoch(a.flags + b, a.epoch);
    return;
  }
  b -= n_logits;
  if (b < a.T) {
    const uint16_t* xr = a.x + (size_t)b * a.H;
    if (FMT == 1)
      quant_row_nvfp4<uint16_t, GSM>(xr, a.H, tid, sm.red, true, a.xq + (size_t)b * (a.H / 2),
                                     a.xs + (size_t)b * (a.H / 16), a.xg + b, nullptr, a.gs_val);
    else
      quant_row_mxfp8<uint16_t>(xr, a.H, tid, true, a.xq + (size_t)b * a.H, a.xs + (size_t)b * (a.H / 32));
    return;
  }
  b -= a.T;
  if (b < n_topk) {
    // tokens 4b .. 4b+3, one per wave, all in token group 4b / (16 MT)
    const int tg = (4 * b) / (16 * MT);
    const bool ok = wait_epoch_flags(a.flags + (size_t)tg * a.S * nex, a.S * nex, a.epoch);
    const int t = 4 * b + (tid >> 6);
    if (t < a.T) {
      router_topk_token<NPER, true>(a.z, a.S, a.T, a.E, a.bias, a.k, a.norm_topk, a.routed_scale, a.ids, a.w,
                                    a.near_tie, t, tid & 63);
      if (!ok && (tid & 63) < a.k)
        __hip_atomic_store(a.w + (size_t)t * a.k + (tid & 63), __builtin_nanf(""), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    publish_epoch(a.flags + n_logits + b, a.epoch);
    return;
  }
  // the dispatch, after every top-k item
  (void)wait_epoch_flags(a.flags + n_logits, n_topk, a.epoch);
  disp_small_body256(a.ids, a.T * a.k, a.E_begin, a.E_local, a.tile_m, a.d.offsets, a.d.sorted, a.d.pos,
                     a.d.worklist, a.d.ntiles, sm.d);
}

int route_prep_flag_words(int E) { return 8 * ((E + 15) / 16) + 64; }

int launch_route_prep(const RoutePrepArgs& a, int fmt, int gs_mode, hipStream_t stream) {
  if (a.T <= 0 || a.T > kRoutePrepMaxTokens || a.T * a.k > kSmallP) return -1;
  const int mt = a.T <= 16 ? 1 : a.T <= 32 ? 2 : 4;
  const int nex = (a.E + 15) / 16;
  const int ntg = (a.T + 16 * mt - 1) / (16 * mt);
  const int items = nex * a.S * ntg + a.T + (a.T + 3) / 4 + 1;
  const int nper = a.E <= 64 ? 1 : a.E <= 128 ? 2 : a.E <= 256 ? 4 : a.E <= 512 ? 8 : 16;
#define MOE_RP(F, G, M, N) hipLaunchKernelGGL((k_route_prep<F, G, M, N>), dim3(items), dim3(256), 0, stream, a)
#define MOE_RP_N(F, G, M)                  \
  do {                                      \
    if (nper == 1) MOE_RP(F, G, M, 1);      \
    else if (nper == 2) MOE_RP(F, G, M, 2); \
    else if (nper == 4) MOE_RP(F, G, M, 4); \
    else if (nper == 8) MOE_RP(F, G, M, 8); \
    else MOE_RP(F, G, M, 16);               \
  } while (0)
#define MOE_RP_M(F, G)                 \
  do {                                 \
    if (mt == 1) MOE_RP_N(F, G, 1);    \
    else if (mt == 2) MOE_RP_N(F, G, 2); \
    else MOE_RP_N(F, G, 4);            \
  } while (0)
  if (fmt == 2) MOE_RP_M(2, GS_ROW);
  else if (gs_mode == GS_STATIC) MOE_RP_M(1, GS_STATIC);
  else MOE_RP_M(1, GS_ROW);
#undef MOE_RP_M
#undef MOE_RP_N
#undef MOE_RP
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Small batches, one launch for two independent steps of the forward:
// workgroup 0 dispatches the pairs, workgroups 1.. quantize the bf16 token
// rows (4 rows each, one per group of 256 threads).
template <int FMT, int GSM>
__global__ __launch_bounds__(1024) void k_prep_small(const uint16_t* __restrict__ x, int T, int H,
                                                     uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                     float* __restrict__ xg, const int32_t* __restrict__ ids,
                                                     int P, int E_begin, int E_local, int tile_m,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                                     int32_t* __restrict__ pos, int32_t* __restrict__ worklist,
                                                     int32_t* __restrict__ ntiles, int32_t* __restrict__ zero,
                                                     int nzero, const float* __restrict__ gs_in, float gs_val) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < nzero; i += 1024) zero[i] = 0;
    disp_small_body(ids, P, E_begin, E_local, tile_m, offsets, sorted, pos, worklist, ntiles);
    return;
  }
  __shared__ float red[4][4];
  const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
  const int row = (blockIdx.x - 1) * 4 + grp;
  const bool live = row < T;
  const int rr = live ? row : T - 1;   // every group takes the barrier; only live rows write
  const uint16_t* xr = x + (size_t)rr * H;
  if (FMT == 1)
    quant_row_nvfp4<uint16_t, GSM>(xr, H, t, red[grp], live, xq + (size_t)rr * (H / 2), xs + (size_t)rr * (H / 16),
                                   xg + rr, gs_in, gs_val);
  else
    quant_row_mxfp8<uint16_t>(xr, H, t, live, xq + (size_t)rr * H, xs + (size_t)rr * (H / 32));
}

int launch_prep_small(int fmt, const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs, float* xg,
                      const int32_t* ids, int P, int E_begin, int E_local, int tile_m, const DispatchBufs& b,
                      int32_t* zero, int nzero, hipStream_t stream, const ActGs& ag) {
  if (P > kSmallP || T <= 0) return -1;
  if (zero == nullptr) nzero = 0;
  const dim3 grid(1 + ceil_div(T, 4));
#define MOE_PREP(F, M)                                                                                             \
  hipLaunchKernelGGL((k_prep_small<F, M>), grid, dim3(1024), 0, stream, x, T, H, xq, xs, xg, ids, P, E_begin,   \
                     E_local, tile_m, b.offsets, b.sorted, b.pos, b.worklist, b.ntiles, zero, nzero, ag.gs_dev, \
                     ag.gs_val)
  if (fmt == 1) {
    if (ag.mode == GS_TENSOR) MOE_PREP(1, GS_TENSOR);
    else if (ag.mode == GS_STATIC) MOE_PREP(1, GS_STATIC);
    else MOE_PREP(1, GS_ROW);
  } else {
    MOE_PREP(2, GS_ROW);
  }
#undef MOE_PREP
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dispatch(const int32_t* ids, int P, int E_begin, int E_local, int tile_m,
                    const DispatchBufs& b, hipStream_t stream) {
  if (P <= kSmallP) {
    hipLaunchKernelGGL(k_disp_small, dim3(1), dim3(1024), 0, stream, ids, P, E_begin, E_local, tile_m, b.offsets,
                       b.sorted, b.pos, b.worklist, b.ntiles);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int chunk = dispatch_chunk(P > 0 ? P : 1);
  const int nchunks = P > 0 ? ceil_div(P, chunk) : 0;
  const size_t lds = (size_t)E_local * sizeof(int32_t);
  int32_t* totals = b.counts + (size_t)(nchunks > 0 ? nchunks : 1) * E_local;
  if (nchunks > 0)
    hipLaunchKernelGGL(k_disp_count, dim3(nchunks), dim3(256), lds, stream, ids, P, chunk, E_begin,
                       E_local, b.counts);
  hipLaunchKernelGGL(k_disp_scan, dim3(E_local), dim3(1024), 0, stream, b.counts, nchunks, E_local,
                     totals);
  hipLaunchKernelGGL(k_disp_offsets, dim3(1), dim3(1024), 0, stream, totals, E_local, tile_m,
                     b.offsets, b.worklist, b.ntiles);
  if (nchunks > 0)
    hipLaunchKernelGGL(k_disp_scatter, dim3(nchunks), dim3(256), lds, stream, ids, P, chunk, E_begin,
                       E_local, b.counts, b.offsets, b.sorted, b.pos);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
