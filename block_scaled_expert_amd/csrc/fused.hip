// The expert half of the layer as one launch (small batches): gate/up GEMM +
// capped SwiGLU, h quantization, down GEMM and the combine run as work items
// of a single kernel instead of four launches -- the single-launch fused MoE
// of the pages (SGLang blog "SGLang and Miles Add Day-0 Support for Inkling 2
// Small", "Performance"; SGLang cookbook "Inkling-2-Small" section 2,
// "MegaMoE": dispatch, the two expert GEMMs and combine in one kernel).
//
// Work items, in queue order:
//   gate/up  (work-list entry, 32 h columns)   entries x F/32
//   down     (work-list entry, 64 y columns)   entries x H/64
//   combine  (token, 1024 columns)             T x ceil(H/1024)
// One workgroup per item: each takes the next item index from a device
// counter when it starts.  An item waits only for items earlier in the queue:
//   - the last gate/up item of an entry to finish quantizes the entry's h
//     rows (NVFP4; MXFP8 h is encoded by each gate/up item) and marks the
//     entry ready;
//   - a down item waits for its entry's ready mark;
//   - combine items wait for the count of finished down items.
// Every item a wait depends on was taken earlier by a running workgroup, so
// the launch drains whatever number of workgroups the chip keeps resident;
// each wait is also bounded (a wait that runs out sets an error word and
// goes on, so every wave reaches the end).  (A persistent grid of resident
// workgroups looping over the items was slower: it drains its loads between
// items and claims unevenly across CUs, where the hardware dispatcher
// spreads a grid and overlaps one workgroup's end with the next one's start.)
//
// The tile bodies are the ones of the separate GEMM kernels (gemm_tile.h),
// the h quantization is the NVFP4 row definition (quant_row.h) and the
// combine the fixed-order sum (combine.h): the output is bit-identical to
// the four-launch chain.  Cross-XCD visibility: each XCD has its own L2.
// Results another workgroup reads (h, its codes and scales, y) are stored
// at device scope (written through, never left dirty in an L2); each wave
// waits for its stores to complete before the workgroup barrier that
// precedes the completion count, so the count needs no L2 write-back (a
// release fence here wrote back the whole L2 per item and cost more than
// the GEMMs).  A consumer invalidates its stale lines (device-scope
// acquire) after the count or flag it waits for.
#include "gemm_tile.h"
#include "quant_row.h"
#include "combine.h"

namespace moe {

namespace {

constexpr int kCtlHead = 0, kCtlDownDone = 1, kCtlErr = 2, kCtlFixed = 4;
constexpr uint32_t kSpinLimit = 1u << 20;     // polls (>= 60 ns each) before a wait gives up

__device__ inline int atomic_add_relaxed(int32_t* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread: wait until *p >= target, then acquire (device scope).  A
// wait that runs out of polls sets *err; once *err is set every wait returns
// at once, so a broken dependency costs one bounded wait, not one per item.
__device__ inline void wait_at_least(int32_t* p, int target, int32_t* err) {
  for (uint32_t it = 0;; it++) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
    if (it >= kSpinLimit) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    if ((it & 255) == 255 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroup barrier after which every wave's stores have completed (each
// wave waits for its own; the workgroup barrier alone does not wait for
// stores): with device-scope stores, the workgroup's results are then
// visible to every XCD, and one thread's count or flag publishes them.
__device__ inline void stores_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
}

}  // namespace

// One workgroup per work item.  The grid covers the largest item count the
// launch can have; workgroups past the device-side count exit at once, the
// others take the next item index from the counter when they start.  The
// hardware dispatches them as slots free up, spread over the CUs, and
// overlaps one workgroup's end with the next one's start.
template <int FMT, int MS, int NSTG, int NSTD, bool PACKED>
__global__ __launch_bounds__(256) void k_moe_fused(GemmArgs g, GemmArgs d, FusedArgs f) {
  constexpr int PF = FMT == 1 ? 3 : 2;
  constexpr int TM = 16 * MS;
  __shared__ union {
    TileLds<0, MS> gu;
    TileLds<1, MS> dn;
  } sm;
  __shared__ int s_item, s_last;
  const int tid = threadIdx.x;
  int32_t* const ctl = f.ctl;
  int32_t* const gu_done = ctl + kCtlFixed;
  int32_t* const ready = ctl + kCtlFixed + f.max_tiles;

  const int nt = g.ntiles[0];   // written by the preceding dispatch launch
  const int F = g.F, H = g.H;
  const int nb1 = F / 32, nb2 = H / 64, ncb = (H / 4 + 255) / 256;
  const int n1 = nt * nb1, n2 = nt * nb2;
  const int total = n1 + n2 + f.T * ncb;
  if ((int)blockIdx.x >= total) return;   // exactly `total` workgroups take an item

  if (tid == 0) s_item = atomic_add_relaxed(ctl + kCtlHead, 1);
  __syncthreads();
  const int item = __builtin_amdgcn_readfirstlane(s_item);   // uniform: scalar registers
  if (item < n1) {
    // gate/up + capped SwiGLU (MXFP8: h encoded here)
    const int tile = item / nb1, bx = item - tile * nb1;
    expert_tile<FMT, 0, MS, PF, NSTG, PACKED, true>(g, tile, bx, sm.gu, tid);
    stores_done_barrier();
    if (tid == 0) {
      const bool last =
          __hip_atomic_fetch_add(gu_done + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nb1 - 1;
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other items' h
      s_last = last;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_last)) {
      if constexpr (FMT == 1) {
        // the entry's h rows are complete: quantize them, one row per wave
        const int el = g.worklist[2 * tile], m0 = g.worklist[2 * tile + 1];
        const int row0 = g.offsets[el] + m0;
        const int rows = min(TM, g.offsets[el + 1] - row0);
        const int wave = tid >> 6, lane = tid & 63;
        for (int m = wave; m < rows; m += 4) {
          const size_t r = (size_t)(row0 + m);
          quant_row_nvfp4_wave<float>(f.h + r * F, F, lane, f.hq + r * (F / 2), f.hs + r * (F / 16), f.hg + r);
        }
        stores_done_barrier();
      }
      if (tid == 0) __hip_atomic_store(ready + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (item < n1 + n2) {
    const int i2 = item - n1, tile = i2 / nb2, bx = i2 - tile * nb2;
    if (tid == 0) wait_at_least(ready + tile, 1, ctl + kCtlErr);
    __syncthreads();
    expert_tile<FMT, 1, MS, PF, NSTD, PACKED, true>(d, tile, bx, sm.dn, tid);
    stores_done_barrier();
    if (tid == 0) atomic_add_relaxed(ctl + kCtlDownDone, 1);
  } else {
    const int i3 = item - n1 - n2, t = i3 / ncb, cb = i3 - t * ncb;
    if (tid == 0) {
      wait_at_least(ctl + kCtlDownDone, n2, ctl + kCtlErr);
      // a wait that ran out anywhere (a down item's included: it set the
      // word before its count, whose stores completed first) poisons the sum
      s_last = __hip_atomic_load(ctl + kCtlErr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int c = cb * 256 + tid;
    if (c < H / 4) {
      if (__builtin_amdgcn_readfirstlane(s_last) == 0)
        combine_col4<false>(f.y, f.pos, f.topk_w, g.k, H, f.out, t, c);
      else
        reinterpret_cast<uint2*>(f.out + (size_t)t * H)[c] = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
    }
  }
}

int fused_ctl_words(int max_tiles) { return kCtlFixed + 2 * max_tiles; }

namespace {

// *dst = src ? *src : v (one thread).
__global__ void k_put_word(int32_t* __restrict__ dst, const int32_t* __restrict__ src, int32_t v) {
  *dst = src != nullptr ? __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : v;
}

}  // namespace

int launch_fused_status(const int32_t* ctl, int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(k_put_word, dim3(1), dim3(1), 0, stream, err, ctl != nullptr ? ctl + kCtlErr : nullptr, 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fused_force_error(int32_t* ctl, hipStream_t stream) {
  hipLaunchKernelGGL(k_put_word, dim3(1), dim3(1), 0, stream, ctl + kCtlErr, nullptr, 1);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {

template <int FMT, int MS, int NSTG, int NSTD, bool PACKED>
int launch_fused_t(const GemmArgs& g, const GemmArgs& d, const FusedArgs& f, hipStream_t stream) {
  // the largest item count: every work-list entry the bound allows
  const long items = (long)g.max_tiles * (g.F / 32 + g.H / 64) + (long)f.T * ((g.H / 4 + 255) / 256);
  hipLaunchKernelGGL((k_moe_fused<FMT, MS, NSTG, NSTD, PACKED>), dim3((unsigned)items), dim3(256), 0, stream, g, d,
                     f);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int FMT, int MS>
int launch_fused_ms(const GemmArgs& g, const GemmArgs& d, const FusedArgs& f, hipStream_t stream) {
  // Inkling 2 Small: H = 4608 gives 36 k steps = 4 waves x 9 (gate/up);
  // F = 2304 gives 18 = 2 waves x 9 (down)
  const bool fast = g.H == 128 * 9 * 4 && g.F == 128 * 9 * 2;
  if (g.packed) return fast ? launch_fused_t<FMT, MS, 9, 9, true>(g, d, f, stream)
                            : launch_fused_t<FMT, MS, 0, 0, true>(g, d, f, stream);
  return fast ? launch_fused_t<FMT, MS, 9, 9, false>(g, d, f, stream)
              : launch_fused_t<FMT, MS, 0, 0, false>(g, d, f, stream);
}

}  // namespace

int launch_moe_fused(const GemmArgs& g, const GemmArgs& d, const FusedArgs& f, hipStream_t stream) {
  const int ms = g.tile_m / 16;
  if (g.fmt == 1) {
    if (ms == 1) return launch_fused_ms<1, 1>(g, d, f, stream);
    if (ms == 2) return launch_fused_ms<1, 2>(g, d, f, stream);
    if (ms == 4) return launch_fused_ms<1, 4>(g, d, f, stream);
  } else {
    if (ms == 1) return launch_fused_ms<2, 1>(g, d, f, stream);
    if (ms == 2) return launch_fused_ms<2, 2>(g, d, f, stream);
    if (ms == 4) return launch_fused_ms<2, 4>(g, d, f, stream);
  }
  return -1;
}

}  // namespace moe
