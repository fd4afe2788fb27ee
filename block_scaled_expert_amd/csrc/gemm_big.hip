// Grouped expert GEMMs for many rows per expert (prefill chunks, an expert-
// parallel share).  The layer and format sources are those of gemm.hip
// (SGLang cookbook "Inkling-2-Small" section 2, "MegaMoE" and "Checkpoints";
// Miles docs section 5.3).
//
// Both kernels: workgroup of 8 waves, tile of 128 rows (a dispatch work-list
// entry with tile_m = 128) x 256 weight rows, k step 128.
//  - The activation tile of each k step is staged through LDS once per
//    workgroup (double-buffered, one barrier per step), in MFMA lane order
//    so every wavefront store and load is 1 KB contiguous.  NVFP4
//    activations are expanded to f16 (code * block scale, exact) while they
//    are written to LDS; MXFP8 activations stay E4M3 with their E8M0 scales.
//  - Each wave streams its own weight rows straight from HBM into MFMA
//    operand registers through a ring of PF k steps (the packed tile layout:
//    one contiguous kilobyte per wavefront load; the canonical layout works
//    too, with 64-byte row pieces).
//  - Waves form 1 (rows) x 8 (weight rows): each wave owns all 128 rows x 32
//    weight rows, so every weight fragment is loaded (and, for NVFP4,
//    expanded to f16) by exactly one wave and feeds 8 MFMAs.
//  - MXFP8 (k_expert_gemm_big_mx): the gate/up epilogue encodes h to MXFP8
//    directly.  NVFP4 (k_expert_gemm_big_nv): see there.
// Each weight element is fetched once per 128 rows of an expert; the
// activation tile once per 256 weight rows.  Down rows larger in total than
// the last-level cache are written with non-temporal stores (GemmArgs
// stream_out).  Work items (row tile, weight
// tile) are ordered so that the items one XCD runs back to back are
// consecutive row tiles of the same weight tile: the hardware hands
// workgroups to the 8 XCDs round-robin, and each XCD has its own L2.
#include <type_traits>

#include "moe_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int BM = 128, BNW = 256, WAVES = 8;

__device__ inline v8h dq8(uint32_t word, v2h sig2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 0) * sig2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 1) * sig2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 2) * sig2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 3) * sig2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// two E4M3 bytes -> f16 pair {sigma0, sigma1} * 2^-8 (field move, see gemm.hip)
// (the two bytes are first spread to the halves, {b0, 0, b1, 0}, so every
// shift is by an inline constant and no shift amount or selector has to be
// held in a vector register)
__device__ inline v2h sig2_of(uint32_t w) {
  const uint32_t x = (w & 0xFFu) | ((w & 0xFF00u) << 8);
  const uint32_t b = ((x & 0x007F007Fu) << 7) | ((x & 0x00800080u) << 8);
  return __builtin_bit_cast(v2h, b);
}

struct BFrag4 {   // NVFP4 weight fragment: 16 B codes + 2 scale bytes
  v4u q;
  uint32_t sc;
};
struct BFrag8 {   // MXFP8 weight fragment: 32 B codes + 1 scale byte
  v4u lo, hi;
  uint32_t sc;
};

// Activation staging: one thread's quarter of one row for one k step.
struct AStage4 {
  v4u q;        // 32 codes (column group g = quarter)
  uint32_t sc;    // their two scale bytes
};
struct AStage8 {
  v4u lo, hi;   // 32 bytes of the 128-byte step
  uint32_t sc;    // scale byte of this quarter
};

// LDS bytes per buffer: NVFP4 8 row tiles x 4 KB of f16; MXFP8 8 x (2 KB + 64 B).
template <int FMT>
constexpr int abuf_bytes() {
  return FMT == 1 ? 8 * 4096 : 8 * (2048 + 64);
}
// LDS bytes ahead of the activation buffers: the tile rows' token indices
// and (NVFP4) their activation scales.
constexpr int kBigHead = 2 * 4 * BM;

// one fp32 down output; the flag is uniform over the launch
__device__ inline void put_out(const GemmArgs& a, size_t idx, float v) {
  if (a.stream_out) __builtin_nontemporal_store(v, a.out + idx);
  else a.out[idx] = v;
}

}  // namespace

// A work item of a large-M launch: one row tile of an expert (a dispatch
// work-list entry) and one of the nx weight tiles.  Work items are ordered so that the
// items one XCD runs back to back are consecutive row tiles of the same
// weight tile.  Returns false for workgroups beyond the launch's items.
struct BigItem {
  int el, row0, rows, bx;
};
__device__ inline bool big_item(const GemmArgs& a, int nx, BigItem& it) {
  const int nt = a.ntiles[0];
  const int items = nx * nt;
  const int hw = blockIdx.x;
  if (hw >= items) return false;
  const int q8 = items / 8, r8 = items % 8, xcd = hw % 8;
  const int L = xcd * q8 + min(xcd, r8) + hw / 8;
  const int tile = L % nt;
  it.bx = L / nt;
  it.el = a.worklist[2 * tile];
  it.row0 = a.offsets[it.el] + a.worklist[2 * tile + 1];
  it.rows = min(BM, a.offsets[it.el + 1] - it.row0);
  return true;
}

// 16-row sub-tiles that hold rows of the item (an expert's last row tile is
// usually partial); the tile bodies are compiled per count, so a partial
// tile issues neither the loads, the LDS traffic nor the MFMAs of its empty
// sub-tiles.
__device__ inline int big_subtiles(int rows) { return min(8, max(1, (rows + 15) >> 4)); }

// MXFP8: each wave owns all of the tile's rows x 32 weight rows (up to 8 x 2
// scaled-MFMA tiles), so every weight fragment is loaded by exactly one wave
// (with waves as 2 row halves x 4, both halves would load it: 80 instead of
// 48 KB of loads per workgroup and k step).  A wave's 16 h columns of a
// gate/up row are half of an MX block; the block maximum is completed across
// the wave pair through LDS.  Token indices of the tile's rows are in the
// first 512 bytes of `lds`, the activation buffers follow.
template <int STAGE, bool PACKED, int PF, int NSUB>
__device__ __forceinline__ void big_mx_tile(const GemmArgs& a, const BigItem& it, uint8_t* lds) {
  constexpr int ABUF = abuf_bytes<2>();
  const int* tok = reinterpret_cast<const int*>(lds);
  uint8_t* abuf = lds + kBigHead;
  const int el = it.el, row0 = it.row0, rows = it.rows, bx = it.bx;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = STAGE == 0 ? a.H : a.F;
  const int NS = K / 128;
  const int NW = STAGE == 0 ? 2 * a.F : a.H;
  const int row_bytes = K, sc_bytes = K / 32;
  const uint8_t* wexp = a.w_codes + (size_t)el * NW * row_bytes;
  const uint8_t* wsexp = a.w_sc + (size_t)el * NW * sc_bytes;

  // activation staging: wave w stages row tile w, lane l row 16 w + l%16 and
  // quarter aq = l/16 of the k step (32 bytes), so each LDS store of the wave
  // is 1 KB contiguous (bank-conflict free).  Waves past the tile's rows
  // stage copies of its first row (a branch here costs the partial-tile
  // bodies their registers).
  const int ar = 16 * wave + r, aq = g;
  const int at = tok[ar] >= 0 ? tok[ar] : tok[0];
  const uint8_t* acode = a.a_codes + (size_t)at * row_bytes + 32 * aq;
  const uint8_t* asc = a.a_sc + (size_t)at * sc_bytes + aq;
  auto aload = [&](int s, AStage8& st) {
    const v4u* p = reinterpret_cast<const v4u*>(acode + s * 128);
    st.lo = p[0];
    st.hi = p[1];
    st.sc = asc[s * 4];
  };
  auto astore = [&](int buf, const AStage8& st) {
    const int h = aq >> 1, g0 = 2 * (aq & 1);
    uint8_t* T = abuf + buf * ABUF + wave * 2112;
    *reinterpret_cast<v4u*>(T + 1024 * h + (r + 16 * g0) * 16) = st.lo;
    *reinterpret_cast<v4u*>(T + 1024 * h + (r + 16 * (g0 + 1)) * 16) = st.hi;
    T[2048 + r + 16 * aq] = (uint8_t)st.sc;
  };

  // this wave's two column groups: gate/up: the gate group and its up group
  // (h columns bx*128 + 16 w ..); down: weight rows bx*256 + 32 w + 16 c
  const uint8_t* brow[2];
  const uint8_t* bsrow[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int n0 = STAGE == 0 ? c * a.F + bx * 128 + 16 * wave : bx * BNW + 32 * wave + 16 * c;
    if (PACKED) {
      const size_t t0 = (size_t)(n0 / 16) * NS;
      brow[c] = wexp + t0 * 2048 + 16 * lane;
      bsrow[c] = wsexp + t0 * 64 + lane;
    } else {
      brow[c] = wexp + (size_t)(n0 + r) * row_bytes + 16 * g;
      bsrow[c] = wsexp + (size_t)(n0 + r) * sc_bytes + g;
    }
  }
  auto bload = [&](int s, BFrag8* B) {
#pragma unroll
    for (int c = 0; c < 2; c++) {
      if (PACKED) {
        const uint8_t* t = brow[c] + (size_t)s * 2048;
        B[c].lo = *reinterpret_cast<const v4u*>(t);
        B[c].hi = *reinterpret_cast<const v4u*>(t + 1024);
        B[c].sc = bsrow[c][s * 64];
      } else {
        B[c].lo = *reinterpret_cast<const v4u*>(brow[c] + s * 128);
        B[c].hi = *reinterpret_cast<const v4u*>(brow[c] + s * 128 + 64);
        B[c].sc = bsrow[c][s * 4];
      }
    }
  };

  v4f acc[NSUB][2];
#pragma unroll
  for (int i = 0; i < NSUB; i++) acc[i][0] = acc[i][1] = v4f{0, 0, 0, 0};

  auto compute = [&](int buf, const BFrag8* B) {
    const uint8_t* A = abuf + buf * ABUF;
    v8i bv[2];
#pragma unroll
    for (int c = 0; c < 2; c++)
      bv[c] = v8i{(int)B[c].lo.x, (int)B[c].lo.y, (int)B[c].lo.z, (int)B[c].lo.w,
                  (int)B[c].hi.x, (int)B[c].hi.y, (int)B[c].hi.z, (int)B[c].hi.w};
#pragma unroll
    for (int i = 0; i < NSUB; i++) {
      const uint8_t* T = A + i * 2112;
      const v4u lo = *reinterpret_cast<const v4u*>(T + 16 * lane);
      const v4u hi = *reinterpret_cast<const v4u*>(T + 1024 + 16 * lane);
      const v8i av = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int as = T[2048 + lane];
#pragma unroll
      for (int c = 0; c < 2; c++)
        acc[i][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[c], acc[i][c], 0, 0, 0, as, 0,
                                                                     (int)B[c].sc);
    }
  };

  BFrag8 bring[PF][2];
  AStage8 ast[PF];
#pragma unroll
  for (int j = 0; j < PF; j++) {
    bload(min(j, NS - 1), bring[j]);
    aload(min(j, NS - 1), ast[j]);
  }
  astore(0, ast[0]);
  aload(min(PF, NS - 1), ast[0]);
  __syncthreads();
  auto one_step = [&](auto J, int s0) {
    constexpr int j = decltype(J)::value;
    const int step = s0 + j;
    compute(step & 1, bring[j]);
    bload(min(step + PF, NS - 1), bring[j]);
    astore((step + 1) & 1, ast[(j + 1) % PF]);
    aload(min(step + 1 + PF, NS - 1), ast[(j + 1) % PF]);
    lds_barrier();
  };
  for (int s0 = 0; s0 < NS; s0 += PF) {
    one_step(std::integral_constant<int, 0>{}, s0);
    if constexpr (PF > 1) one_step(std::integral_constant<int, 1>{}, s0);
    if constexpr (PF > 2) one_step(std::integral_constant<int, 2>{}, s0);
  }

  // epilogue: acc reg q of lane l in tile (i, c): row 16 i + 4 (l/16) + q,
  // weight row 16 * (group c) + l%16.  The main loop ended with a barrier,
  // so the activation buffers are free for the block maxima.
  const int cl = lane & 15, g4 = lane >> 4;
  if (STAGE == 0) {
    const float inv_c = 1.0f / a.cap;
    float* amx = reinterpret_cast<float*>(abuf);   // [128 rows][8 waves]
    float h[4 * NSUB], u[4 * NSUB];
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        h[4 * i + q] = acc[i][0][q];
        u[4 * i + q] = acc[i][1][q];
      }
    cap_swiglu_n(h, u, a.cap_form, a.cap, inv_c);
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 16 * i + 4 * g4 + q;
        float am = m < rows ? fabsf(h[4 * i + q]) : 0.0f;
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
        if (cl == 0) amx[m * 8 + wave] = am;
      }
    __syncthreads();
    const int col = bx * 128 + 16 * wave + cl;
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 16 * i + 4 * g4 + q;
        if (m >= rows) continue;
        const float am = fmaxf(amx[m * 8 + wave], amx[m * 8 + (wave ^ 1)]);
        const int E = mx_exponent(am);
        a.out_q[(size_t)(row0 + m) * a.F + col] = (uint8_t)mx_encode(h[4 * i + q], pow2f(-E));
        if (cl == 0 && (wave & 1) == 0) a.out_s[(size_t)(row0 + m) * (a.F / 32) + col / 32] = (uint8_t)(E + 127);
      }
  } else {
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 16 * i + 4 * g4 + q;
        if (m >= rows) continue;
#pragma unroll
        for (int c = 0; c < 2; c++) put_out(a, (size_t)(row0 + m) * a.H + bx * BNW + 32 * wave + 16 * c + cl, acc[i][c][q]);
      }
  }
}

template <int STAGE, bool PACKED, int PF>
__global__ __launch_bounds__(512, 4) void k_expert_gemm_big_mx(GemmArgs a) {
  static_assert(PF >= 1 && PF <= 3, "ring depth");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  BigItem it;
  if (!big_item(a, STAGE == 0 ? a.F / 128 : a.H / BNW, it)) return;
  const int tid = threadIdx.x;
  if (tid < BM)
    reinterpret_cast<int*>(lds)[tid] =
        tid < it.rows ? (STAGE == 0 ? a.sorted[it.row0 + tid] / a.k : it.row0 + tid) : -1;
  __syncthreads();
  // 6 or 7 sub-tiles run the full body: the compiler's schedules for those
  // two counts need more than 128 registers
  switch (big_subtiles(it.rows)) {
    case 1: big_mx_tile<STAGE, PACKED, PF, 1>(a, it, lds); break;
    case 2: big_mx_tile<STAGE, PACKED, PF, 2>(a, it, lds); break;
    case 3: big_mx_tile<STAGE, PACKED, PF, 3>(a, it, lds); break;
    case 4: big_mx_tile<STAGE, PACKED, PF, 4>(a, it, lds); break;
    case 5: big_mx_tile<STAGE, PACKED, PF, 5>(a, it, lds); break;
    default: big_mx_tile<STAGE, PACKED, PF, 8>(a, it, lds); break;
  }
}

// NVFP4: the same tile (128 rows x 256 weight rows, 8 waves, k step 128,
// activations expanded to f16 once per workgroup in LDS), waves 1 (rows) x 8
// (weight rows): each wave owns all of the tile's rows x 32 weight rows (up
// to 8 x 2 MFMA tiles).  The exact NVFP4 path is limited by vector-ALU issue
// (operand expansion shares issue slots with the MFMAs); here every weight
// fragment is expanded once per workgroup and feeds up to 8 MFMAs, for twice
// the LDS reads of a 2 x 4 arrangement (about half of gfx950's LDS bandwidth
// at the MFMA rate).  One step of weights in flight and a scheduling barrier
// between the four 32-wide parts of a step keep the kernel within 128
// registers, so two workgroups (16 waves) share a CU and cover each other's
// latency.  `lds` starts with the rows' token indices (512 bytes) and
// activation scales (512 bytes); the activation buffers follow.
template <int STAGE, bool PACKED, int PF, int NSUB>
__device__ __forceinline__ void big_nv_tile(const GemmArgs& a, const BigItem& it, uint8_t* lds) {
  constexpr int ABUF = abuf_bytes<1>();
  int* tok = reinterpret_cast<int*>(lds);
  float* rgs = reinterpret_cast<float*>(lds + 4 * BM);
  uint8_t* abuf = lds + kBigHead;
  const int el = it.el, row0 = it.row0, rows = it.rows, bx = it.bx;

  // the wave index is uniform: readfirstlane puts it (and every address
  // derived from it alone) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = STAGE == 0 ? a.H : a.F;
  const int NS = K / 128;
  const int NW = STAGE == 0 ? 2 * a.F : a.H;
  const int row_bytes = K / 2, sc_bytes = K / 16;
  const uint8_t* wexp = a.w_codes + (size_t)el * NW * row_bytes;
  const uint8_t* wsexp = a.w_sc + (size_t)el * NW * sc_bytes;

  // this wave's two column groups of 16 weight rows: gate/up: the gate group
  // and its up group (h columns bx*128 + 16 w ..); down: rows bx*256 + 32 w + 16 c
  // (uniform row bases in scalar registers, one 32-bit lane offset each for
  // codes and scales)
  const uint8_t* brow[2];
  const uint8_t* bsrow[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int n0 = STAGE == 0 ? c * a.F + bx * 128 + 16 * wave : bx * BNW + 32 * wave + 16 * c;
    if (PACKED) {
      const size_t t0 = (size_t)(n0 / 16) * NS;
      brow[c] = wexp + t0 * 1024;
      bsrow[c] = wsexp + t0 * 128;
    } else {
      brow[c] = wexp + (size_t)n0 * row_bytes;
      bsrow[c] = wsexp + (size_t)n0 * sc_bytes;
    }
  }
  const uint32_t boff = PACKED ? 16 * lane : r * row_bytes + 16 * g;
  const uint32_t bsoff = PACKED ? 2 * lane : r * sc_bytes + 2 * g;
  auto bload = [&](int s, BFrag4* B) {
#pragma unroll
    for (int c = 0; c < 2; c++) {
      B[c].q = *reinterpret_cast<const v4u*>(brow[c] + (PACKED ? (size_t)s * 1024 : (size_t)s * 64) + boff);
      B[c].sc = *reinterpret_cast<const uint16_t*>(bsrow[c] + (PACKED ? s * 128 : s * 8) + bsoff);
    }
  };

  v4f acc[NSUB][2];
#pragma unroll
  for (int i = 0; i < NSUB; i++) acc[i][0] = acc[i][1] = v4f{0, 0, 0, 0};

  // One k step on activation buffer `buf`, scheduled by hand as 4 x NSUB
  // chunks (part j of the step's four 32-wide parts, row sub-tile i), each
  // fenced by a scheduling barrier.  Chunk (j, i) issues the LDS read of the
  // next chunk's activation fragment, its own two MFMAs, and an even share
  // of the vector-ALU work: the expansion of part j+1's weight fragments
  // (8 convert + multiply pairs per part) and, when STG, of part j of the
  // next activation tile (4 pairs in the part's last two chunks, then one
  // LDS store into buffer `nbuf`).
  // The matrix cores then never wait behind a block of conversions.
  // `issue_loads` runs at the start of part 3, once this step's weight
  // fragments are no longer read.
  auto compute = [&](int buf, const BFrag4* B, int nbuf, const AStage4& st, auto STG, auto&& issue_loads) {
    constexpr bool stage_here = decltype(STG)::value;
    constexpr int NC = 4 * NSUB;
    const uint8_t* A = abuf + buf * ABUF + lane * 16;
    uint8_t* S = abuf + nbuf * ABUF + wave * 4096 + lane * 16;
    v2h bs[2][2], as[2];
#pragma unroll
    for (int c = 0; c < 2; c++) {
      const v2h sp = sig2_of(B[c].sc);
      bs[c][0] = v2h{sp[0], sp[0]};
      bs[c][1] = v2h{sp[1], sp[1]};
    }
    if constexpr (stage_here) {
      const v2h sp = sig2_of(st.sc);
      as[0] = v2h{sp[0], sp[0]};
      as[1] = v2h{sp[1], sp[1]};
    }
    auto word = [](const v4u& q, int j) { return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w; };
    // f16 pair p (codes 2p, 2p+1) of word w times the scale pair
    auto pair = [](uint32_t w, int p, v2h sc) {
      const v2h f = p == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0)
                  : p == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1)
                  : p == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
      return f * sc;
    };
    auto pack = [](const v2h (&x)[4]) {
      return v8h{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
    };
    // gate/up: a wave in its k step issues ahead of the waves in the step
    // barrier, loads or epilogue (prefill gate/up 4.79 -> 4.68 ms on one
    // box; the down kernel did not gain)
    if constexpr (STAGE == 0) __builtin_amdgcn_s_setprio(1);
    v2h bx[2][2][4];   // [part parity][column group][pair]
    v2h sx[4];
#pragma unroll
    for (int c = 0; c < 2; c++)
#pragma unroll
      for (int p = 0; p < 4; p++) bx[0][c][p] = pair(word(B[c].q, 0), p, bs[c][0]);
    constexpr int AR = 3;   // activation fragments in flight: reads run two chunks ahead
    v8h av[AR];
#pragma unroll
    for (int t = 0; t < AR - 1 && t < NC; t++)
      av[t] = *reinterpret_cast<const v8h*>(A + (t % NSUB) * 4096 + (t / NSUB) * 1024);
#pragma unroll
    for (int t = 0; t < NC; t++) {
      const int j = t / NSUB, i = t % NSUB;
      __builtin_amdgcn_sched_barrier(0);
      if (t == 3 * NSUB) issue_loads();
      if (t + AR - 1 < NC) {
        const int tn = t + AR - 1, jn = tn / NSUB, in = tn % NSUB;
        av[tn % AR] = *reinterpret_cast<const v8h*>(A + in * 4096 + jn * 1024);
      }
      const v8h b0 = pack(bx[j & 1][0]), b1 = pack(bx[j & 1][1]);
      acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t % AR], b0, acc[i][0], 0, 0, 0);
      acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t % AR], b1, acc[i][1], 0, 0, 0);
      if (j < 3) {
#pragma unroll
        for (int k = 0; k < 8; k++)
          if (k * NSUB / 8 == i) bx[(j + 1) & 1][k >> 2][k & 3] = pair(word(B[k >> 2].q, j + 1), k & 3, bs[k >> 2][(j + 1) >> 1]);
      }
      if constexpr (stage_here) {
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (NSUB - 2 + k / 2 == i) sx[k] = pair(word(st.q, j), k, as[j >> 1]);
        if (i == NSUB - 1) *reinterpret_cast<v8h*>(S + j * 1024) = pack(sx);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STAGE == 0) __builtin_amdgcn_s_setprio(0);
  };

  // main loop: PF steps of weights and activations in flight (as in
  // big_mx_tile; ring slots are compile-time constants).  Full tiles stage
  // the next activation tile inside compute; partial tiles (only the first
  // NSUB waves stage) after it.
  // Prologue: the tile rows' token indices (threads < 128), then the first
  // weight steps, which do not depend on them (memory operations complete in
  // issue order, so the index loads are not held up), then the indices are
  // published through LDS.  The row scales are needed only by the epilogue:
  // their loads stay in flight through the main loop.
  // (No load sits under a branch -- the compiler would drain every
  // outstanding load where the branch joins -- so every thread loads an
  // index of the tile, clamped to its last row, and selects afterwards.)
  const int m_own = min(tid % BM, rows - 1);
  const int tk_any = STAGE == 0 ? a.sorted[row0 + m_own] / a.k : row0 + m_own;
  BFrag4 bring[PF][2];
#pragma unroll
  for (int j = 0; j < PF; j++) bload(min(j, NS - 1), bring[j]);
  const bool own_row = tid < BM && tid < rows;
  if (tid < BM) tok[tid] = own_row ? tk_any : -1;
  const float gs_any = a.a_gs[tk_any];
  lds_barrier();

  // activation staging as in big_mx_tile (wave w < NSUB: row tile w; NVFP4
  // expanded to f16 on the way into LDS)
  const bool stager = NSUB == 8 || wave < NSUB;
  const int ar = 16 * wave + r, aq = g;
  const int at = tok[ar] >= 0 ? tok[ar] : tok[0];
  const uint8_t* acode = a.a_codes + (size_t)at * row_bytes + 16 * aq;
  const uint8_t* asc = a.a_sc + (size_t)at * sc_bytes + 2 * aq;
  auto aload = [&](int s, AStage4& st) {
    if (!stager) return;
    st.q = *reinterpret_cast<const v4u*>(acode + s * 64);
    st.sc = *reinterpret_cast<const uint16_t*>(asc + s * 8);
  };
  auto astore = [&](int buf, const AStage4& st) {
    if (!stager) return;
    const v2h sp = sig2_of(st.sc);
    const v2h s0 = v2h{sp[0], sp[0]}, s1 = v2h{sp[1], sp[1]};
    uint8_t* base = abuf + buf * ABUF + wave * 4096 + lane * 16;
    *reinterpret_cast<v8h*>(base + 0 * 1024) = dq8(st.q.x, s0);
    *reinterpret_cast<v8h*>(base + 1 * 1024) = dq8(st.q.y, s0);
    *reinterpret_cast<v8h*>(base + 2 * 1024) = dq8(st.q.z, s1);
    *reinterpret_cast<v8h*>(base + 3 * 1024) = dq8(st.q.w, s1);
  };

  AStage4 ast[PF];
#pragma unroll
  for (int j = 0; j < PF; j++) aload(min(j, NS - 1), ast[j]);
  astore(0, ast[0]);
  aload(min(PF, NS - 1), ast[0]);
  lds_barrier();
  auto one_step = [&](auto J, int s0) {
    constexpr int j = decltype(J)::value;
    const int step = s0 + j;
    AStage4& nst = ast[(j + 1) % PF];
    // with one step in flight the next weights reuse this step's ring slot,
    // loaded once part 3 runs; deeper rings load after the step
    auto next_b = [&] { if constexpr (PF == 1) bload(min(step + PF, NS - 1), bring[j]); };
    if constexpr (NSUB == 8) {
      compute(step & 1, bring[j], (step + 1) & 1, nst, std::true_type{}, next_b);
    } else {
      compute(step & 1, bring[j], (step + 1) & 1, nst, std::false_type{}, next_b);
      astore((step + 1) & 1, nst);
    }
    if constexpr (PF > 1) bload(min(step + PF, NS - 1), bring[j]);
    aload(min(step + 1 + PF, NS - 1), nst);
    lds_barrier();
  };
  for (int s0 = 0; s0 < NS; s0 += PF) {
    one_step(std::integral_constant<int, 0>{}, s0);
    if constexpr (PF > 1) one_step(std::integral_constant<int, 1>{}, s0);
    if constexpr (PF > 2) one_step(std::integral_constant<int, 2>{}, s0);
  }

  // row scales into LDS for the epilogue (the main loop's last barrier has
  // passed: nothing reads that LDS any more)
  if (tid < BM) rgs[tid] = own_row ? gs_any : 0.0f;
  lds_barrier();

  // epilogue: acc reg q of lane l in tile (i, c): row 16 i + 4 (l/16) + q,
  // weight row 16 * (group c) + l%16
  const int cl = lane & 15, g4 = lane >> 4;
  if (STAGE == 0) {
    const float inv_c = 1.0f / a.cap;
    const ScalePair wg = split_scale(a.w_gs[3 * el + 0]), wu = split_scale(a.w_gs[3 * el + 1]);
    const int col = bx * 128 + 16 * wave + cl;
    float h[4 * NSUB], u[4 * NSUB];
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const ScalePair ga = split_scale(rgs[16 * i + 4 * g4 + q]);
        h[4 * i + q] = apply_scale(acc[i][0][q], ga * wg);
        u[4 * i + q] = apply_scale(acc[i][1][q], ga * wu);
      }
    cap_swiglu_n(h, u, a.cap_form, a.cap, inv_c);
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 16 * i + 4 * g4 + q;
        if (m >= rows) continue;
        a.out[(size_t)(row0 + m) * a.F + col] = h[4 * i + q];
      }
  } else {
    const ScalePair wd = split_scale(a.w_gs[3 * el + 2]);
#pragma unroll
    for (int i = 0; i < NSUB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 16 * i + 4 * g4 + q;
        if (m >= rows) continue;
        const ScalePair hs = split_scale(rgs[m]) * wd;
#pragma unroll
        for (int c = 0; c < 2; c++)
          put_out(a, (size_t)(row0 + m) * a.H + bx * BNW + 32 * wave + 16 * c + cl, apply_scale(acc[i][c][q], hs));
      }
  }
}

template <int STAGE, bool PACKED, int PF>
__global__ __launch_bounds__(512, 4) void k_expert_gemm_big_nv(GemmArgs a) {
  static_assert(PF >= 1 && PF <= 3, "ring depth");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  BigItem it;
  if (!big_item(a, STAGE == 0 ? a.F / 128 : a.H / BNW, it)) return;
  switch (big_subtiles(it.rows)) {
    case 1: big_nv_tile<STAGE, PACKED, PF, 1>(a, it, lds); break;
    case 2: big_nv_tile<STAGE, PACKED, PF, 2>(a, it, lds); break;
    case 3: big_nv_tile<STAGE, PACKED, PF, 3>(a, it, lds); break;
    case 4: big_nv_tile<STAGE, PACKED, PF, 4>(a, it, lds); break;
    case 5: big_nv_tile<STAGE, PACKED, PF, 5>(a, it, lds); break;
    case 6: big_nv_tile<STAGE, PACKED, PF, 6>(a, it, lds); break;
    case 7: big_nv_tile<STAGE, PACKED, PF, 7>(a, it, lds); break;
    default: big_nv_tile<STAGE, PACKED, PF, 8>(a, it, lds); break;
  }
}


namespace {

template <int ST, bool PK, int PF>
void launch_mx_one(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  const size_t lds = kBigHead + 2 * abuf_bytes<2>();
  hipLaunchKernelGGL((k_expert_gemm_big_mx<ST, PK, PF>), grid, dim3(WAVES * 64), lds, stream, a);
}

template <int ST, bool PK, int PF>
void launch_nv_one(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  const size_t lds = kBigHead + 2 * abuf_bytes<1>();
  // dynamic LDS of 64 KiB and more must be allowed explicitly; set on every
  // launch (a host-side call) so no state is shared across threads or devices
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_expert_gemm_big_nv<ST, PK, PF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((k_expert_gemm_big_nv<ST, PK, PF>), grid, dim3(WAVES * 64), lds, stream, a);
}

template <int FMT, int ST, bool PK>
void launch_pf(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  // One step of weights in flight per wave: both kernels then fit 128
  // registers, so two workgroups (16 waves) share a CU and hide each other's
  // latency -- faster than deeper rings at one workgroup per CU (same-box
  // A/B: EP share gate/up 258 -> 222 us, prefill gate/up 6.32 -> 5.77 ms).
  if constexpr (FMT == 1) launch_nv_one<ST, PK, 1>(a, grid, stream);
  else launch_mx_one<ST, PK, 1>(a, grid, stream);
}

}  // namespace

bool gemm_big_supported(int H, int F) { return H % BNW == 0 && F % 128 == 0; }

int launch_gemm_big(const GemmArgs& a, int stage, hipStream_t stream) {
  // one workgroup per work item, at most (weight tiles) x (work-list bound)
  const int nx = stage == 0 ? a.F / 128 : a.H / BNW;
  const dim3 grid(nx * a.max_tiles);
#define MOE_BIG(FMT, ST)                                     \
  do {                                                       \
    if (a.packed) launch_pf<FMT, ST, true>(a, grid, stream); \
    else launch_pf<FMT, ST, false>(a, grid, stream);         \
  } while (0)
  if (a.fmt == 2) {
    if (stage == 0) MOE_BIG(2, 0); else MOE_BIG(2, 1);
  } else {
    if (stage == 0) MOE_BIG(1, 0); else MOE_BIG(1, 1);
  }
#undef MOE_BIG
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
