// Grouped expert GEMMs for work-list entries of 16 to 64 rows: one
// workgroup per (entry, 64-row weight slice); the tile body and its design
// notes are in gemm_tile.h.
#include "gemm_tile.h"

namespace moe {

// grid.y walks the work list (entries past the device-side count exit at
// once), grid.x the 64-row slices of the expert's weight matrix.
template <int FMT, int STAGE, int MS, int PF, int NST, bool PACKED>
__global__ __launch_bounds__(256) void k_expert_gemm(GemmArgs a) {
  __shared__ TileLds<STAGE, MS> sm;
  const int tile = blockIdx.y;
  if (tile >= a.ntiles[0]) return;
  expert_tile<FMT, STAGE, MS, PF, NST, PACKED>(a, tile, blockIdx.x, sm, threadIdx.x);
}

int gemm_tile_m(int T, int k, int E) {
  // expected rows per expert (uniform routing) picks the rows per work-list
  // entry; 128-row entries go to the LDS-tiled kernel (gemm_big.hip)
  const long avg = (long)T * k / (E > 0 ? E : 1);
  return avg <= 2 ? 16 : avg <= 24 ? 32 : avg <= 48 ? 64 : 128;
}

static int launch_any(const GemmArgs& a, int stage, hipStream_t stream) {
  if (a.tile_m == 128) return launch_gemm_big(a, stage, stream);
  const dim3 block(256);
  const dim3 grid(stage == 0 ? a.F / 32 : a.H / 64, a.max_tiles);
  // Inkling 2 Small: H = 4608 gives 36 k steps = 4 waves x 9 (gate/up);
  // F = 2304 gives 18 = 2 waves x 9 (down).
  const bool fast = stage == 0 ? a.H == 128 * 9 * 4 : a.F == 128 * 9 * 2;
#define MOE_LAUNCH(FMT, ST, MS, NST)                                                                \
  do {                                                                                              \
    if (a.packed)                                                                                   \
      hipLaunchKernelGGL((k_expert_gemm<FMT, ST, MS, (FMT == 1 ? 3 : 2), NST, true>), grid, block, 0, \
                         stream, a);                                                                \
    else                                                                                            \
      hipLaunchKernelGGL((k_expert_gemm<FMT, ST, MS, (FMT == 1 ? 3 : 2), NST, false>), grid, block, 0, \
                         stream, a);                                                                \
  } while (0)
#define MOE_LAUNCH_N(FMT, ST, MS)                  \
  do {                                             \
    if (fast) MOE_LAUNCH(FMT, ST, MS, 9);          \
    else MOE_LAUNCH(FMT, ST, MS, 0);               \
  } while (0)
#define MOE_LAUNCH_MS(FMT, ST)                        \
  do {                                                \
    if (a.tile_m == 16) MOE_LAUNCH_N(FMT, ST, 1);     \
    else if (a.tile_m == 32) MOE_LAUNCH_N(FMT, ST, 2); \
    else MOE_LAUNCH_N(FMT, ST, 4);                    \
  } while (0)
  if (a.fmt == 2) {
    if (stage == 0) MOE_LAUNCH_MS(2, 0); else MOE_LAUNCH_MS(2, 1);
  } else {
    if (stage == 0) MOE_LAUNCH_MS(1, 0); else MOE_LAUNCH_MS(1, 1);
  }
#undef MOE_LAUNCH_MS
#undef MOE_LAUNCH_N
#undef MOE_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_gateup(const GemmArgs& a, hipStream_t stream) { return launch_any(a, 0, stream); }
int launch_gemm_down(const GemmArgs& a, hipStream_t stream) { return launch_any(a, 1, stream); }

}  // namespace moe

