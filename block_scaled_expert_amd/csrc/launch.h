// Internal launch wrappers of the MoE kernels (host side).  Argument
// checking happens in api.hip before any of these is called; each wrapper
// only enqueues work and returns 0, or -1 when hipGetLastError reports a
// failed launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Where NVFP4 activation rows take their fp32 scale (enum moe_act_gs):
// mode 0 per row; 1 the tensor's shared scale in the device word gs_dev
// (launch_act_gs_tensor writes it); 2 the fixed value gs_val.
struct ActGs {
  int mode = 0;
  const float* gs_dev = nullptr;
  float gs_val = 1.0f;
};

// Activation quantization of `rows` rows (further limited by *rows_dev when
// non-null) of width `cols`.  fmt: 1 NVFP4, 2 MXFP8 (ag ignored).  dtype: 0
// bf16, 1 fp32.
int launch_quant(int fmt, int dtype, const void* x, int rows, const int* rows_dev, int cols,
                 uint8_t* codes, uint8_t* scales, float* gs, hipStream_t stream, const ActGs& ag = ActGs{});

// The shared NVFP4 scale of a whole [rows][cols] tensor (rows limited by
// *rows_dev when non-null): scratch[0] = max|x| / 2688 (1 for an all-zero
// tensor), with scratch[1 .. 1 + kActGsPartials) holding partial maxima.
constexpr int kActGsPartials = 256;
constexpr size_t kActGsScratchBytes = 4 * (1 + kActGsPartials);
int launch_act_gs_tensor(int dtype, const void* x, int rows, const int* rows_dev, int cols, float* scratch,
                         hipStream_t stream);

// Router: logits into z (fp32 workspace: router_splits(T, E) partial [T][E]
// planes, router_z_rows(max_tokens) * E floats at most), then sigmoid + bias
// + top-k.
int router_splits(int T, int E);
size_t router_z_rows(int max_tokens);
int launch_router(const uint16_t* x, int T, int H, const uint16_t* wr, const float* bias, int E,
                  int k, int norm_topk, float routed_scale, float* z, int32_t* ids, float* w,
                  uint8_t* near_tie, hipStream_t stream);

// Dispatch workspace layout (all int32):
//   counts [nchunks][E_local], totals [E_local], tiles: worklist [max_tiles] int2,
//   ntiles [1].
struct DispatchBufs {
  int32_t* counts;      // [nchunks * E_local]
  int32_t* offsets;     // [E_local + 1]
  int32_t* sorted;      // [P] (nullable)
  int32_t* pos;         // [P] (nullable)
  int32_t* worklist;    // [2 * max_tiles] (nullable): (local expert, first row)
  int32_t* ntiles;      // [1] (nullable)
};
int dispatch_chunk(int P);
int launch_dispatch(const int32_t* ids, int P, int E_begin, int E_local, int tile_m,
                    const DispatchBufs& b, hipStream_t stream);
// Pair counts up to this take one workgroup for the dispatch ...
constexpr int kSmallDispatchPairs = 4096;
// ... and can share a launch with the quantization of the bf16 token rows
// (xq / xs / xg as launch_quant writes them for fmt 1 or 2).
// zero (nullable): nzero int32 words the launch also clears.
int launch_prep_small(int fmt, const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs, float* xg,
                      const int32_t* ids, int P, int E_begin, int E_local, int tile_m, const DispatchBufs& b,
                      int32_t* zero, int nzero, hipStream_t stream, const ActGs& ag = ActGs{});

// Routing, quantization of the token rows and dispatch in one launch for
// small batches (dispatch.hip): T <= kRoutePrepMaxTokens, T k <= 4096.
constexpr int kRoutePrepMaxTokens = 256;
struct RoutePrepArgs {
  // router
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  int T, H, E, k, S, norm_topk;
  float routed_scale;
  float* z;                // router_splits(T, E) partial planes [S][T][E]
  int32_t* ids;
  float* w;
  uint8_t* near_tie;       // nullable
  // quantization (fmt 1: codes, scales, row scales; fmt 2: codes, scales)
  uint8_t* xq;
  uint8_t* xs;
  float* xg;
  float gs_val;            // static NVFP4 scale (gs mode 2)
  // dispatch
  int E_begin, E_local, tile_m;
  DispatchBufs d;
  // completion flags (route_prep_flag_words(E) uint64 words) and the call's epoch
  uint64_t* flags;
  uint64_t epoch;
};
int route_prep_flag_words(int E);
// gs_mode: ActGs mode 0 (per row) or 2 (static); per-tensor scales are not supported here
int launch_route_prep(const RoutePrepArgs& a, int fmt, int gs_mode, hipStream_t stream);

// Weight encoding: nmat matrices [rows][cols] (dtype 0 bf16, 1 fp32) to
// canonical NVFP4 (fmt 1: one fp32 scale per matrix, written to
// gs[(m / gs_group) * gs_stride + m % gs_group]; amax: nmat words of device
// scratch) or MXFP8 (fmt 2), and back to fp32.
int launch_encode_weights(int fmt, int dtype, const void* w, int nmat, int rows, int cols, uint8_t* codes,
                          uint8_t* scales, float* gs, int gs_group, int gs_stride, uint32_t* amax,
                          hipStream_t stream);
int launch_decode_weights(int fmt, const uint8_t* codes, const uint8_t* scales, const float* gs, int nmat, int rows,
                          int cols, int gs_group, int gs_stride, float* out, hipStream_t stream);

struct GemmArgs {
  int fmt;                 // 1 NVFP4, 2 MXFP8
  int H, F, k;
  int E_local;
  // activations (quantized rows)
  const uint8_t* a_codes;  // gate/up: x codes [T][...]; down: h codes [P][...]
  const uint8_t* a_sc;
  const float* a_gs;       // NVFP4 row scales (nullable for MXFP8)
  // weights
  const uint8_t* w_codes;
  const uint8_t* w_sc;
  const float* w_gs;       // [E_local][3] (NVFP4)
  int packed;              // weights in the packed tile layout
  // routing
  const int32_t* offsets;  // [E_local+1]
  const int32_t* sorted;   // [P] pair ids in expert order
  const int32_t* worklist; // [2*max_tiles]
  const int32_t* ntiles;   // [1]
  int max_tiles;           // grid.y: an upper bound of *ntiles
  int tile_m;              // rows per work-list entry (16, 32, 64 or 128; matches dispatch)
  // epilogue
  int cap_form;
  float cap;
  float* out;              // gate/up: h [P][F]; down: y [P][H] (rows in sorted order)
  // MXFP8 gate/up only: h is encoded in the epilogue (each workgroup's
  // columns of a row are whole 32-element blocks) into codes [P][F] and E8M0
  // scales [P][F/32] instead of being written to `out`
  uint8_t* out_q;
  uint8_t* out_s;
  // down only: `out` is larger than the last-level cache, written with
  // non-temporal stores (the combine then streams it back)
  int stream_out;
};
// Buffers above this size (MI355X's 256 MiB last-level cache) are written
// and read back with the non-temporal hint; below it, the consumer finds
// them in the cache.
constexpr size_t kStreamBytes = size_t(256) << 20;
int gemm_tile_m(int T, int k, int E);
// LDS-staged variant for 128-row work-list entries (gemm_big.hip); needs
// H % 256 == 0 and F % 128 == 0.
bool gemm_big_supported(int H, int F);
int launch_gemm_big(const GemmArgs& a, int stage, hipStream_t stream);
int launch_gemm_gateup(const GemmArgs& a, hipStream_t stream);
int launch_gemm_down(const GemmArgs& a, hipStream_t stream);

// The expert half as one launch (fused.hip) for work-list entries
// of 16 to 64 rows.  ctl: fused_ctl_words(max_tiles) int32 words, zero when
// the launch starts (the quantize + dispatch launch before it clears them).
struct FusedArgs {
  int32_t* ctl;
  int max_tiles;
  // NVFP4 h quantization per sorted row: fp32 h in; codes, scales, row scales out
  const float* h;
  uint8_t* hq;
  uint8_t* hs;
  float* hg;
  // combine
  const float* y;
  const int32_t* pos;
  const float* topk_w;
  int T;
  uint16_t* out;
};
int fused_ctl_words(int max_tiles);
int launch_moe_fused(const GemmArgs& g, const GemmArgs& d, const FusedArgs& f, hipStream_t stream);
// *err = the single launch's error word (ctl non-null) or 0 (ctl null)
int launch_fused_status(const int32_t* ctl, int32_t* err, hipStream_t stream);
// sets the error word (after the launch that clears it): every wait returns at once
int launch_fused_force_error(int32_t* ctl, hipStream_t stream);

// The epilogue's capped SwiGLU on n fp32 pairs (moe_cap_swiglu).
int launch_cap_swiglu(int form, float cap, const float* g, const float* u, long n, float* h, hipStream_t stream);

// Repack nmat canonical [N][K] matrices (codes + scales) into the packed
// tile layout (moe_prepare_weights).
int launch_pack(int fmt, const uint8_t* codes, const uint8_t* scales, long nmat, int N, int K,
                uint8_t* pcodes, uint8_t* pscales, hipStream_t stream);

int launch_combine(const float* y, const int32_t* pos, const float* w, int T, int k, int H, bool nt,
                   uint16_t* out, hipStream_t stream);

}  // namespace moe
