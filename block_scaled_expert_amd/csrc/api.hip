// C ABI of the MoE library (include/moe.h): argument checking, the gfx950
// check, workspace carving and the launch sequence.  Nothing here allocates,
// frees or synchronizes; every launch goes on the caller's stream.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>

#include "../../include/moe.h"
#include "launch.h"
#include "moe_common.h"

using namespace moe;

namespace {

// Per-device result of the architecture check: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_arch_ok[64];

int device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED_DEVICE;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    v = moe_check_arch(prop.gcnArchName) == MOE_OK ? 1 : -1;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

int n_local(const moe_config* c) { return c->num_local_experts; }

// Workspace regions (byte offsets, each 256-byte aligned).
struct Layout {
  size_t z, xq, xs, xg, ags, counts, offsets, sorted, pos, work, ntiles, ctl, flags, h, hq, hs, hg, y, total;
  int max_tiles, nchunks;
};

Layout layout(const moe_config* c, int T) {
  Layout L;
  const size_t H = c->hidden, F = c->ffn, E = c->num_experts, EL = n_local(c), k = c->top_k;
  const size_t P = (size_t)T * k;
  const bool nv = c->fmt == MOE_FMT_NVFP4;
  L.nchunks = P > 0 ? ceil_div((long)P, dispatch_chunk((int)P)) : 0;
  L.max_tiles = ceil_div((long)P, 16) + (int)EL;   // smallest tile_m is 16
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.z = take(router_z_rows(T) * E * 4);
  L.xq = take((size_t)T * (nv ? H / 2 : H));
  L.xs = take((size_t)T * (nv ? H / 16 : H / 32));
  L.xg = take((size_t)T * 4);
  L.ags = take(nv ? kActGsScratchBytes : 0);   // NVFP4 per-tensor scale: partial maxima + the scale
  // dispatch never uses more than 1024 chunks (see dispatch_chunk)
  L.counts = take((size_t)(1024 + 1) * EL * 4);
  L.offsets = take((EL + 1) * 4);
  L.sorted = take(P * 4);
  L.pos = take(P * 4);
  L.work = take((size_t)L.max_tiles * 2 * 4);
  L.ntiles = take(4);
  L.ctl = take((size_t)fused_ctl_words(L.max_tiles) * 4);
  L.flags = take((size_t)route_prep_flag_words((int)E) * 8);   // moe_route_forward's completion flags
  L.h = take(nv ? P * F * 4 : 0);    // fp32 h: NVFP4 only (MXFP8 h is encoded by the gate/up epilogue)
  L.hq = take(P * (nv ? F / 2 : F));
  L.hs = take(P * (nv ? F / 16 : F / 32));
  L.hg = take(nv ? P * 4 : 0);
  L.y = take(P * H * 4);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_ws(const moe_config* c, int T, void* ws, size_t ws_bytes) {
  if (T > c->max_tokens) return MOE_ERR_TOO_MANY_TOKENS;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < layout(c, c->max_tokens).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

void record(void* const* ev, int idx, hipStream_t s) {
  if (ev != nullptr && ev[idx] != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(ev[idx]), s);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Rows per work-list entry of a forward of T tokens.
int forward_tile_m(const moe_config* c, int T) {
  int tile_m = gemm_tile_m(T, c->top_k, c->num_experts);
  if (tile_m == 128 && !gemm_big_supported(c->hidden, c->ffn)) tile_m = 64;
  return tile_m;
}

// Whether moe_forward_fused runs its single expert-half launch for T tokens:
// at most 4096 pairs (the one-launch quantize + dispatch), entries of at most
// 64 rows, and NVFP4 activation scales per row (a per-tensor h scale needs
// every h row before any is quantized).
bool fused_applies(const moe_config* c, int T) {
  const long P = (long)T * c->top_k;
  const bool nv = c->fmt == MOE_FMT_NVFP4;
  return T > 0 && P <= kSmallDispatchPairs && forward_tile_m(c, T) <= 64 &&
         (!nv || c->act_gs == MOE_ACT_GS_PER_ROW);
}

// Where the NVFP4 activation rows of site 0 (x) / 1 (h) take their scale.
ActGs act_gs_of(const moe_config* c, int site, float* scratch) {
  ActGs a;
  if (c->fmt != MOE_FMT_NVFP4) return a;
  if (c->act_gs == MOE_ACT_GS_PER_TENSOR) {
    a.mode = 1;
    a.gs_dev = scratch;
  } else if (c->act_gs == MOE_ACT_GS_STATIC) {
    a.mode = 2;
    a.gs_val = c->act_gs_static[site];
  }
  return a;
}

// Workspace of moe_forward_noalloc: a file-scope device array, one per GPU
// the library runs on, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device array: host code only ever
// uses the device address hipGetSymbolAddress returns for the current
// device (scratch_ptr).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // per device, set once under g_scratch_mu

// Device address of the current device's scratch array (nullptr on error).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Per-call epochs for moe_route_forward's completion flags: distinct for
// every call in the process and, through a random start, unlikely to match
// anything a workspace held before.
std::atomic<uint64_t> g_epoch{0};
std::once_flag g_epoch_once;
uint64_t next_epoch() {
  std::call_once(g_epoch_once, [] {
    std::random_device rd;
    g_epoch.store(((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ 0x9E3779B97F4A7C15ull);
  });
  uint64_t e;
  do e = g_epoch.fetch_add(1) + 1; while (e == 0);
  return e;
}

// Whether moe_route_forward runs routing, x quantization and dispatch as
// one launch: small batches (T <= 256, T k <= 4096) without a per-tensor
// NVFP4 x scale (which needs its maximum before any row).
bool route_forward_one_launch(const moe_config* c, int T) {
  return T > 0 && T <= kRoutePrepMaxTokens && (long)T * c->top_k <= kSmallDispatchPairs &&
         !(c->fmt == MOE_FMT_NVFP4 && c->act_gs == MOE_ACT_GS_PER_TENSOR);
}

bool test_fail_requested() {
  const char* v = std::getenv("MOE_FUSED_TEST_FAIL");
  return v != nullptr && v[0] == '1';
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_TOO_MANY_TOKENS: return "more tokens than the configured maximum";
    case MOE_ERR_UNSUPPORTED_FORMAT: return "unsupported expert format";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH_TOO_SMALL: return "batch needs more than moe_forward_noalloc's 64 MiB scratch buffer";
    default: return "unknown status";
  }
}

int moe_check_arch(const char* arch) {
  if (arch == nullptr) return MOE_ERR_INVALID_ARG;
  if (std::strncmp(arch, "gfx950", 6) != 0) return MOE_ERR_UNSUPPORTED_DEVICE;
  const char n = arch[6];
  return (n == '\0' || n == ':') ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

int moe_validate_config(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->fmt != MOE_FMT_NVFP4 && c->fmt != MOE_FMT_MXFP8) return MOE_ERR_UNSUPPORTED_FORMAT;
  if (c->hidden <= 0 || c->hidden % 128 != 0 || c->hidden > (1 << 16)) return MOE_ERR_INVALID_ARG;
  if (c->ffn <= 0 || c->ffn % 128 != 0 || c->ffn > (1 << 16)) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts > 1024) return MOE_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > 32 || c->top_k > c->num_experts) return MOE_ERR_INVALID_ARG;
  if (c->expert_begin < 0 || c->num_local_experts < 1 ||
      c->expert_begin + c->num_local_experts > c->num_experts)
    return MOE_ERR_INVALID_ARG;
  if (c->cap_form < MOE_CAP_SOFT_GATE_UP || c->cap_form > MOE_CAP_NONE) return MOE_ERR_INVALID_ARG;
  if (c->cap_form != MOE_CAP_NONE && !(c->cap > 0.0f)) return MOE_ERR_INVALID_ARG;
  if (c->max_tokens < 0 || (long)c->max_tokens * c->top_k > (1L << 26)) return MOE_ERR_INVALID_ARG;
  if (c->act_gs < MOE_ACT_GS_PER_ROW || c->act_gs > MOE_ACT_GS_STATIC) return MOE_ERR_INVALID_ARG;
  if (c->act_gs == MOE_ACT_GS_STATIC && c->fmt == MOE_FMT_NVFP4)
    for (int i = 0; i < 2; i++)   // positive, finite, and 6 * 448 * gs stays finite
      if (!(c->act_gs_static[i] > 0.0f && c->act_gs_static[i] <= 0x1p120f)) return MOE_ERR_INVALID_ARG;
  // the GEMM work list rides grid.y (at most 65535 entries)
  if (ceil_div((long)c->max_tokens * c->top_k, 16) + c->num_local_experts > 65535) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int moe_workspace_size(const moe_config* c, size_t* bytes) {
  const int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = layout(c, c->max_tokens).total;
  return MOE_OK;
}

int moe_quantize_act(const moe_config* c, int32_t site, int32_t dtype, const void* x, int32_t rows, int32_t cols,
                     uint8_t* codes, uint8_t* scales, float* row_gs, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  const int fmt = c->fmt;
  if (site != 0 && site != 1) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16)) return MOE_ERR_INVALID_ARG;
  const bool nv = fmt == MOE_FMT_NVFP4;
  if (nv && (row_gs == nullptr || !aligned(row_gs, 4))) return MOE_ERR_INVALID_ARG;
  const bool tensor = nv && c->act_gs == MOE_ACT_GS_PER_TENSOR;
  if (tensor) {
    if (ws == nullptr || !aligned(ws, 4)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < kActGsScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  if ((st = device_check()) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int bad = 0;
  if (tensor) bad |= launch_act_gs_tensor(dtype, x, rows, nullptr, cols, static_cast<float*>(ws), s);
  bad |= launch_quant(fmt, dtype, x, rows, nullptr, cols, codes, scales, row_gs, s,
                      act_gs_of(c, site, static_cast<float*>(ws)));
  return bad ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_cap_swiglu(const moe_config* c, const float* g, const float* u, int64_t n, float* h, void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (g == nullptr || u == nullptr || h == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(g, 4) || !aligned(u, 4) || !aligned(h, 4)) return MOE_ERR_INVALID_ARG;
  if ((st = device_check()) != MOE_OK) return st;
  const float cap = c->cap_form == MOE_CAP_NONE ? 1.0f : c->cap;
  return launch_cap_swiglu(c->cap_form, cap, g, u, (long)n, h, static_cast<hipStream_t>(stream)) == 0
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

int moe_encode_weights(int32_t fmt, int32_t dtype, const void* w, int32_t nmat, int32_t rows, int32_t cols,
                       uint8_t* codes, uint8_t* scales, float* gs, int32_t gs_group, int32_t gs_stride,
                       void* ws, size_t ws_bytes, void* stream) {
  if (fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_MXFP8) return MOE_ERR_UNSUPPORTED_FORMAT;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
  if (nmat < 0 || rows <= 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if ((long)nmat * rows > (1L << 30) || (long)nmat * rows * cols > (1L << 40)) return MOE_ERR_INVALID_ARG;
  if (nmat == 0) return MOE_OK;
  if (w == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(codes, 16)) return MOE_ERR_INVALID_ARG;
  if (fmt == MOE_FMT_NVFP4) {
    if (gs == nullptr || gs_group < 1 || gs_stride < gs_group || ws == nullptr || !aligned(ws, 4))
      return MOE_ERR_INVALID_ARG;
    if (ws_bytes < (size_t)nmat * 4) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  const int d = device_check();
  if (d != MOE_OK) return d;
  return launch_encode_weights(fmt, dtype, w, nmat, rows, cols, codes, scales, gs, gs_group, gs_stride,
                               static_cast<uint32_t*>(ws), static_cast<hipStream_t>(stream)) == 0
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

int moe_decode_weights(int32_t fmt, const uint8_t* codes, const uint8_t* scales, const float* gs,
                       int32_t gs_group, int32_t gs_stride, int32_t nmat, int32_t rows, int32_t cols, float* out,
                       void* stream) {
  if (fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_MXFP8) return MOE_ERR_UNSUPPORTED_FORMAT;
  if (nmat < 0 || rows <= 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if ((long)nmat * rows > (1L << 30) || (long)nmat * rows * cols > (1L << 40)) return MOE_ERR_INVALID_ARG;
  if (nmat == 0) return MOE_OK;
  if (codes == nullptr || scales == nullptr || out == nullptr || !aligned(codes, 8)) return MOE_ERR_INVALID_ARG;
  if (fmt == MOE_FMT_NVFP4 && (gs == nullptr || gs_group < 1 || gs_stride < gs_group)) return MOE_ERR_INVALID_ARG;
  const int d = device_check();
  if (d != MOE_OK) return d;
  return launch_decode_weights(fmt, codes, scales, gs, nmat, rows, cols, gs_group, gs_stride, out,
                               static_cast<hipStream_t>(stream)) == 0
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

int moe_route(const moe_config* c, const void* x, int32_t T, const void* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, uint8_t* near_tie, void* ws, size_t ws_bytes,
              void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, T, ws, ws_bytes)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || bias == nullptr || topk_ids == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(bias, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = device_check()) != MOE_OK) return st;
  const Layout L = layout(c, c->max_tokens);
  return launch_router(static_cast<const uint16_t*>(x), T, c->hidden, static_cast<const uint16_t*>(w_router),
                       bias, c->num_experts, c->top_k, c->norm_topk, c->routed_scale, at<float>(ws, L.z),
                       topk_ids, topk_w, near_tie, static_cast<hipStream_t>(stream)) == 0
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

int moe_dispatch(const moe_config* c, const int32_t* topk_ids, int32_t T, int32_t* expert_offsets,
                 int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0 || expert_offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (T > 0 && topk_ids == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_pairs, 4) || !aligned(pair_pos, 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, T, ws, ws_bytes)) != MOE_OK) return st;
  if ((st = device_check()) != MOE_OK) return st;
  const Layout L = layout(c, c->max_tokens);
  DispatchBufs b{};
  b.counts = at<int32_t>(ws, L.counts);
  b.offsets = expert_offsets;
  b.sorted = sorted_pairs;
  b.pos = pair_pos;
  b.worklist = nullptr;
  b.ntiles = nullptr;
  return launch_dispatch(topk_ids, T * c->top_k, c->expert_begin, c->num_local_experts, 32, b,
                         static_cast<hipStream_t>(stream)) == 0
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

int moe_prepare_weights(const moe_config* c, const moe_expert_weights* src, moe_expert_weights* dst,
                        void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (src == nullptr || dst == nullptr) return MOE_ERR_INVALID_ARG;
  if (src->layout != MOE_LAYOUT_CANONICAL) return MOE_ERR_INVALID_ARG;
  if (src->w13 == nullptr || src->w13_sc == nullptr || src->w2 == nullptr || src->w2_sc == nullptr ||
      dst->w13 == nullptr || dst->w13_sc == nullptr || dst->w2 == nullptr || dst->w2_sc == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (src->w13 == dst->w13 || src->w2 == dst->w2 || src->w13_sc == dst->w13_sc || src->w2_sc == dst->w2_sc)
    return MOE_ERR_INVALID_ARG;
  for (const moe_expert_weights* w : {src, static_cast<const moe_expert_weights*>(dst)})
    if (!aligned(w->w13, 16) || !aligned(w->w2, 16) || !aligned(w->w13_sc, 4) || !aligned(w->w2_sc, 4))
      return MOE_ERR_INVALID_ARG;
  if ((st = device_check()) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long n = c->num_local_experts;
  int bad = launch_pack(c->fmt, src->w13, src->w13_sc, n, 2 * c->ffn, c->hidden, const_cast<uint8_t*>(dst->w13),
                        const_cast<uint8_t*>(dst->w13_sc), s);
  bad |= launch_pack(c->fmt, src->w2, src->w2_sc, n, c->hidden, c->ffn, const_cast<uint8_t*>(dst->w2),
                     const_cast<uint8_t*>(dst->w2_sc), s);
  if (bad) return MOE_ERR_LAUNCH;
  dst->layout = MOE_LAYOUT_PACKED;
  return MOE_OK;
}

static int forward_impl(const moe_config* c, const void* x, int32_t T, const int32_t* topk_ids,
                        const float* topk_w, const moe_expert_weights* w, void* out, void* ws, size_t ws_bytes,
                        void* stream, void* const* events, bool fused, bool prep_done = false) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, T, ws, ws_bytes)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || w == nullptr || out == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (w->w13 == nullptr || w->w13_sc == nullptr || w->w2 == nullptr || w->w2_sc == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (c->fmt == MOE_FMT_NVFP4 && w->gs == nullptr) return MOE_ERR_INVALID_ARG;
  if (w->layout != MOE_LAYOUT_CANONICAL && w->layout != MOE_LAYOUT_PACKED) return MOE_ERR_INVALID_ARG;
  // the kernels' 16-byte vector loads and stores
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w->w13, 16) || !aligned(w->w2, 16) ||
      !aligned(w->w13_sc, 4) || !aligned(w->w2_sc, 4) || !aligned(w->gs, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = device_check()) != MOE_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout L = layout(c, c->max_tokens);
  const int H = c->hidden, F = c->ffn, k = c->top_k, EL = c->num_local_experts;
  const int P = T * k;
  const bool nv = c->fmt == MOE_FMT_NVFP4;
  int bad = 0;

  const int tile_m = forward_tile_m(c, T);
  DispatchBufs b{};
  b.counts = at<int32_t>(ws, L.counts);
  b.offsets = at<int32_t>(ws, L.offsets);
  b.sorted = at<int32_t>(ws, L.sorted);
  b.pos = at<int32_t>(ws, L.pos);
  b.worklist = at<int32_t>(ws, L.work);
  b.ntiles = at<int32_t>(ws, L.ntiles);
  // the single launch covers work-list entries of 16 to 64 rows after
  // the one-launch quantize + dispatch (which also clears its control words)
  fused = fused && fused_applies(c, T);
  float* const ags = at<float>(ws, L.ags);
  const ActGs agx = act_gs_of(c, 0, ags), agh = act_gs_of(c, 1, ags);
  if (prep_done) {
    // x quantized and dispatched by moe_route_forward's first launch
  } else if (P <= kSmallDispatchPairs) {
    // 1 + 2. quantize x per row and dispatch (+ tile list) in one launch; the
    // quantize-x stage covers both, the dispatch stage is empty
    record(events, 2 * MOE_STAGE_QUANT_X, s);
    if (agx.mode == 1) bad |= launch_act_gs_tensor(0, x, T, nullptr, H, ags, s);
    bad |= launch_prep_small(c->fmt, static_cast<const uint16_t*>(x), T, H, at<uint8_t>(ws, L.xq),
                             at<uint8_t>(ws, L.xs), at<float>(ws, L.xg), topk_ids, P, c->expert_begin, EL, tile_m,
                             b, fused ? at<int32_t>(ws, L.ctl) : nullptr,
                             fused ? fused_ctl_words(L.max_tiles) : 0, s, agx);
    if (fused && test_fail_requested()) bad |= launch_fused_force_error(at<int32_t>(ws, L.ctl), s);
    record(events, 2 * MOE_STAGE_QUANT_X + 1, s);
    record(events, 2 * MOE_STAGE_DISPATCH, s);
    record(events, 2 * MOE_STAGE_DISPATCH + 1, s);
  } else {
    // 1. quantize x per row
    record(events, 2 * MOE_STAGE_QUANT_X, s);
    if (agx.mode == 1) bad |= launch_act_gs_tensor(0, x, T, nullptr, H, ags, s);
    bad |= launch_quant(c->fmt, 0, x, T, nullptr, H, at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs),
                        at<float>(ws, L.xg), s, agx);
    record(events, 2 * MOE_STAGE_QUANT_X + 1, s);
    // 2. dispatch + tile list
    record(events, 2 * MOE_STAGE_DISPATCH, s);
    bad |= launch_dispatch(topk_ids, P, c->expert_begin, EL, tile_m, b, s);
    record(events, 2 * MOE_STAGE_DISPATCH + 1, s);
  }

  // 3. gate/up GEMM + capped SwiGLU -> h (fp32, sorted rows)
  GemmArgs g{};
  g.fmt = c->fmt;
  g.H = H;
  g.F = F;
  g.k = k;
  g.E_local = EL;
  g.a_codes = at<uint8_t>(ws, L.xq);
  g.a_sc = at<uint8_t>(ws, L.xs);
  g.a_gs = at<float>(ws, L.xg);
  g.w_codes = w->w13;
  g.w_sc = w->w13_sc;
  g.w_gs = w->gs;
  g.packed = w->layout == MOE_LAYOUT_PACKED;
  g.offsets = b.offsets;
  g.sorted = b.sorted;
  g.worklist = b.worklist;
  g.ntiles = b.ntiles;
  g.max_tiles = ceil_div((long)P, tile_m) + EL;
  g.tile_m = tile_m;
  g.cap_form = c->cap_form;
  g.cap = c->cap_form == MOE_CAP_NONE ? 1.0f : c->cap;
  const bool fuse_h = c->fmt == MOE_FMT_MXFP8;   // MXFP8 h is encoded by the gate/up epilogue
  g.out = fuse_h ? nullptr : at<float>(ws, L.h);
  g.out_q = fuse_h ? at<uint8_t>(ws, L.hq) : nullptr;
  g.out_s = fuse_h ? at<uint8_t>(ws, L.hs) : nullptr;

  // down GEMM arguments
  GemmArgs d = g;
  d.a_codes = at<uint8_t>(ws, L.hq);
  d.a_sc = at<uint8_t>(ws, L.hs);
  d.a_gs = fuse_h ? nullptr : at<float>(ws, L.hg);
  d.w_codes = w->w2;
  d.w_sc = w->w2_sc;
  d.out = at<float>(ws, L.y);
  // y larger than the last-level cache streams (non-temporal stores in the
  // down epilogue, loads in the combine); its size is taken at the expected
  // local pair count, the one the tile height follows
  const size_t y_bytes = (size_t)T * k * EL / c->num_experts * H * sizeof(float);
  const bool stream_y = y_bytes > kStreamBytes;
  d.stream_out = stream_y ? 1 : 0;

  if (fused) {
    // 3-6 in one launch, timed by the GATE_UP pair
    FusedArgs f{};
    f.ctl = at<int32_t>(ws, L.ctl);
    f.max_tiles = g.max_tiles;
    f.h = at<float>(ws, L.h);
    f.hq = at<uint8_t>(ws, L.hq);
    f.hs = at<uint8_t>(ws, L.hs);
    f.hg = at<float>(ws, L.hg);
    f.y = at<float>(ws, L.y);
    f.pos = b.pos;
    f.topk_w = topk_w;
    f.T = T;
    f.out = static_cast<uint16_t*>(out);
    record(events, 2 * MOE_STAGE_GATE_UP, s);
    bad |= launch_moe_fused(g, d, f, s);
    record(events, 2 * MOE_STAGE_GATE_UP + 1, s);
    for (int st = MOE_STAGE_QUANT_H; st <= MOE_STAGE_COMBINE; st++) {
      record(events, 2 * st, s);
      record(events, 2 * st + 1, s);
    }
    return bad ? MOE_ERR_LAUNCH : MOE_OK;
  }

  record(events, 2 * MOE_STAGE_GATE_UP, s);
  bad |= launch_gemm_gateup(g, s);
  record(events, 2 * MOE_STAGE_GATE_UP + 1, s);

  // 4. quantize h per (token, expert) row (NVFP4: the row scale needs the
  // whole row, so a kernel of its own; the row count lives on the device)
  record(events, 2 * MOE_STAGE_QUANT_H, s);
  if (!fuse_h) {
    if (agh.mode == 1) bad |= launch_act_gs_tensor(1, at<float>(ws, L.h), P, b.offsets + EL, F, ags, s);
    bad |= launch_quant(c->fmt, 1, at<float>(ws, L.h), P, b.offsets + EL, F, at<uint8_t>(ws, L.hq),
                        at<uint8_t>(ws, L.hs), at<float>(ws, L.hg), s, agh);
  }
  record(events, 2 * MOE_STAGE_QUANT_H + 1, s);

  // 5. down GEMM -> y (fp32, sorted rows)
  record(events, 2 * MOE_STAGE_DOWN, s);
  bad |= launch_gemm_down(d, s);
  record(events, 2 * MOE_STAGE_DOWN + 1, s);

  // 6. combine
  record(events, 2 * MOE_STAGE_COMBINE, s);
  bad |= launch_combine(at<float>(ws, L.y), b.pos, topk_w, T, k, H, stream_y, static_cast<uint16_t*>(out), s);
  record(events, 2 * MOE_STAGE_COMBINE + 1, s);
  (void)nv;
  return bad ? MOE_ERR_LAUNCH : MOE_OK;
}

int moe_forward(const moe_config* c, const void* x, int32_t T, const int32_t* topk_ids, const float* topk_w,
                const moe_expert_weights* w, void* out, void* ws, size_t ws_bytes, void* stream,
                void* const* events) {
  return forward_impl(c, x, T, topk_ids, topk_w, w, out, ws, ws_bytes, stream, events, false);
}

int moe_forward_fused(const moe_config* c, const void* x, int32_t T, const int32_t* topk_ids,
                      const float* topk_w, const moe_expert_weights* w, void* out, void* ws, size_t ws_bytes,
                      void* stream, void* const* events) {
  return forward_impl(c, x, T, topk_ids, topk_w, w, out, ws, ws_bytes, stream, events, true);
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_forward_noalloc(const moe_config* c, const void* x, int32_t T, const int32_t* topk_ids, const float* topk_w,
                        const moe_expert_weights* w, void* out, void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > c->max_tokens) return MOE_ERR_TOO_MANY_TOKENS;
  if (T == 0) return MOE_OK;
  // the workspace layout sized for this call's T, carved from the array
  moe_config ct = *c;
  ct.max_tokens = T;
  if (layout(&ct, T).total > kScratchBytes) return MOE_ERR_SCRATCH_TOO_SMALL;
  if ((st = device_check()) != MOE_OK) return st;
  void* ws = scratch_ptr();
  if (ws == nullptr) return MOE_ERR_HIP;
  return forward_impl(&ct, x, T, topk_ids, topk_w, w, out, ws, kScratchBytes, stream, nullptr, false);
}

int moe_route_forward(const moe_config* c, const void* x, int32_t T, const void* w_router, const float* bias,
                      int32_t* topk_ids, float* topk_w, uint8_t* near_tie, const moe_expert_weights* w, void* out,
                      void* ws, size_t ws_bytes, void* stream, void* const* events) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, T, ws, ws_bytes)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const bool nv = c->fmt == MOE_FMT_NVFP4;
  const bool one_launch = route_forward_one_launch(c, T);
  if (!one_launch) {
    // larger batches: the router launches, then moe_forward's sequence
    if ((st = moe_route(c, x, T, w_router, bias, topk_ids, topk_w, near_tie, ws, ws_bytes, stream)) != MOE_OK)
      return st;
    return forward_impl(c, x, T, topk_ids, topk_w, w, out, ws, ws_bytes, stream, events, false);
  }
  if (x == nullptr || w_router == nullptr || bias == nullptr || topk_ids == nullptr || topk_w == nullptr ||
      w == nullptr || out == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(bias, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = device_check()) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout L = layout(c, c->max_tokens);
  RoutePrepArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wr = static_cast<const uint16_t*>(w_router);
  a.bias = bias;
  a.T = T;
  a.H = c->hidden;
  a.E = c->num_experts;
  a.k = c->top_k;
  a.S = router_splits(T, c->num_experts);
  a.norm_topk = c->norm_topk;
  a.routed_scale = c->routed_scale;
  a.z = at<float>(ws, L.z);
  a.ids = topk_ids;
  a.w = topk_w;
  a.near_tie = near_tie;
  a.xq = at<uint8_t>(ws, L.xq);
  a.xs = at<uint8_t>(ws, L.xs);
  a.xg = at<float>(ws, L.xg);
  a.gs_val = (nv && c->act_gs == MOE_ACT_GS_STATIC) ? c->act_gs_static[0] : 1.0f;
  a.E_begin = c->expert_begin;
  a.E_local = c->num_local_experts;
  a.tile_m = forward_tile_m(c, T);
  a.d.counts = at<int32_t>(ws, L.counts);
  a.d.offsets = at<int32_t>(ws, L.offsets);
  a.d.sorted = at<int32_t>(ws, L.sorted);
  a.d.pos = at<int32_t>(ws, L.pos);
  a.d.worklist = at<int32_t>(ws, L.work);
  a.d.ntiles = at<int32_t>(ws, L.ntiles);
  a.flags = at<uint64_t>(ws, L.flags);
  a.epoch = next_epoch();
  record(events, 2 * MOE_STAGE_QUANT_X, s);
  const int bad = launch_route_prep(a, c->fmt, (nv && c->act_gs == MOE_ACT_GS_STATIC) ? 2 : 0, s);
  record(events, 2 * MOE_STAGE_QUANT_X + 1, s);
  record(events, 2 * MOE_STAGE_DISPATCH, s);
  record(events, 2 * MOE_STAGE_DISPATCH + 1, s);
  if (bad) return MOE_ERR_LAUNCH;
  return forward_impl(c, x, T, topk_ids, topk_w, w, out, ws, ws_bytes, stream, events, false, true);
}

int moe_forward_fused_status(const moe_config* c, int32_t T, const void* ws, size_t ws_bytes, int32_t* err,
                             void* stream) {
  int st = moe_validate_config(c);
  if (st != MOE_OK) return st;
  if (T < 0 || err == nullptr || !aligned(err, 4)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(c, T, const_cast<void*>(ws), ws_bytes)) != MOE_OK) return st;
  if ((st = device_check()) != MOE_OK) return st;
  const Layout L = layout(c, c->max_tokens);
  const int32_t* ctl = fused_applies(c, T) ? at<int32_t>(const_cast<void*>(ws), L.ctl) : nullptr;
  return launch_fused_status(ctl, err, static_cast<hipStream_t>(stream)) == 0 ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
