// Tile body of the grouped expert GEMMs on gfx950 MFMA for work-list entries
// of 16 to 64 rows (the two expert GEMMs of the SGLang cookbook's MegaMoE
// description, section 2; W4A4 / W8A8 per Miles docs section 5.3; the expert
// layout of the NVFP4 / MXFP8 checkpoint, SGLang cookbook section 2
// "Checkpoints").  Used by the per-GEMM kernels (gemm.hip) and by the
// single-launch expert-half kernel (fused.hip).
//
// Work: the dispatch work list holds one entry per (local expert, block of
// TM = 16*MS sorted rows); one tile is one entry x one 64-row slice of the
// expert's weight matrix.  Each workgroup's 4 waves split K; every wave loads its
// weight slice straight from HBM into MFMA operand registers (no LDS on the
// weight path: each weight byte is used by exactly one wave), the partial
// tiles meet in LDS and are summed in a fixed order, and the epilogue
// applies the fp32 scales and writes the output rows in sorted order.
//
// MXFP8 (W8A8): v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands and the
//   E8M0 block scales as the instruction's scale operands -- exact products.
//   Operand layout (measured on gfx950): lane l holds row l%16; its bytes
//   0-15 are k = 16*(l/16) + i and bytes 16-31 are k = 64 + 16*(l/16) + i;
//   its scale byte applies to k-block l/16 (k in [32*(l/16), +32)).  With
//   the natural memory order that is two 16-byte loads at k0 + 16g and
//   k0 + 64 + 16g and the scale of block k0/32 + g.
// NVFP4 (W4A4): NVFP4's E4M3 scale per 16 cannot ride the E8M0-per-32 scale
//   operand, and E2M1 times an E4M3 scale needs up to 6 significant bits, so
//   both operands are expanded in registers to f16 = E2M1 value * block
//   scale (exact: at most 6 bits, magnitudes 2^-10 .. 2688) and multiplied
//   on v_mfma_f32_16x16x32_f16 (products exact in the fp32 accumulator).
//   The two fp32 tensor/row scales are applied in the epilogue.  Each lane
//   loads 16 bytes = 32 consecutive E2M1 codes per 128-wide k step and feeds
//   8 of them to each of four MFMAs; both operands use the same k mapping.
#pragma once

#include <type_traits>

#include "moe_common.h"
#include "launch.h"

namespace moe {

// E2M1 x 8 (one 32-bit word, low nibble first) -> f16 x 8, each times its
// block scale.  The convert applies the power of two 2^8 (its scale operand
// only contributes an exponent); the block scale enters as sigma * 2^-8 in
// f16 (see sig_pair), so every product is exactly E2M1 * sigma: at most 6
// significant bits, magnitudes 2^-10 .. 2688, all normal f16 numbers.
__device__ inline v8h dequant8(uint32_t word, v2h sig2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 0) * sig2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 1) * sig2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 2) * sig2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 3) * sig2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two E4M3 scale bytes (low 16 bits of w) -> f16 pair {sigma0, sigma1} * 2^-8.
// Moving the E4M3 exponent/mantissa field 7 bits up lands it in the f16
// exponent/mantissa field with the bias difference 8 = 15 - 7, so the f16
// bit pattern is the E4M3 value times 2^-8, subnormals included.
__device__ inline v2h sig_pair(uint32_t w) {
  const uint32_t b = ((w & 0x7Fu) << 7) | ((w & 0x80u) << 8) | ((w & 0x7F00u) << 15) | ((w & 0x8000u) << 16);
  return __builtin_bit_cast(v2h, b);
}

// One k step (128 elements) of operand data for one 16-row group.
struct Frag8 {            // MXFP8: 32 bytes + scale byte
  uint4 lo, hi;
  uint32_t sc;
};
struct Frag4 {            // NVFP4: 16 bytes + two scale bytes
  uint4 q;
  uint32_t sc;
};

// Fragment loads.  Weights are streamed once per step: their loads carry the
// non-temporal hint (no allocation priority in the caches, which on this
// chip raises a plain read stream from about 6.4 to 7.1 TB/s); activation
// rows, re-read by every column block, are loaded normally.
template <bool NT, typename T>
__device__ inline T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ inline uint4 as_uint4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

template <bool NT = false>
__device__ inline void load_frag(Frag8& f, const uint8_t* row, const uint8_t* sc_row, int k0, int g) {
  f.lo = as_uint4(ld<NT>(reinterpret_cast<const v4u*>(row + k0 + 16 * g)));
  f.hi = as_uint4(ld<NT>(reinterpret_cast<const v4u*>(row + k0 + 64 + 16 * g)));
  f.sc = ld<NT>(sc_row + k0 / 32 + g);
}
template <bool NT = false>
__device__ inline void load_frag(Frag4& f, const uint8_t* row, const uint8_t* sc_row, int k0, int g) {
  f.q = as_uint4(ld<NT>(reinterpret_cast<const v4u*>(row + k0 / 2 + 16 * g)));
  const uint8_t* s = sc_row + k0 / 16 + 2 * g;
  f.sc = (uint32_t)ld<NT>(s) | ((uint32_t)ld<NT>(s + 1) << 8);
}
// Packed layout (weights only): tile = 16 rows x 128 columns in MFMA lane
// order; `tile` points at lane 0 of the row group's step-0 tile, sc at its
// scales.
__device__ inline void load_frag_packed(Frag8& f, const uint8_t* tile, const uint8_t* sc, int step, int lane) {
  const uint8_t* t = tile + (size_t)step * 2048 + 16 * lane;
  f.lo = as_uint4(ld<true>(reinterpret_cast<const v4u*>(t)));
  f.hi = as_uint4(ld<true>(reinterpret_cast<const v4u*>(t + 1024)));
  f.sc = ld<true>(sc + step * 64 + lane);
}
__device__ inline void load_frag_packed(Frag4& f, const uint8_t* tile, const uint8_t* sc, int step, int lane) {
  f.q = as_uint4(ld<true>(reinterpret_cast<const v4u*>(tile + (size_t)step * 1024 + 16 * lane)));
  f.sc = ld<true>(reinterpret_cast<const uint16_t*>(sc + step * 128 + 2 * lane));
}

__device__ inline void zero_frag(Frag8& f) {
  f.lo = make_uint4(0, 0, 0, 0);
  f.hi = f.lo;
  f.sc = 127;
}
__device__ inline void zero_frag(Frag4& f) {
  f.q = make_uint4(0, 0, 0, 0);
  f.sc = 0x3838;  // 1.0, 1.0
}

__device__ inline v4f mma(const Frag8& a, const Frag8& b, v4f c) {
  const v8i av = v8i{(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w,
                     (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
  const v8i bv = v8i{(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w,
                     (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, (int)a.sc, 0, (int)b.sc);
}

// NVFP4: expand a fragment into four f16 MFMA operands.
struct Half4 {
  v8h v[4];
};
__device__ inline void expand(const Frag4& f, Half4& h) {
  const v2h sp = sig_pair(f.sc);
  const v2h s0 = v2h{sp[0], sp[0]}, s1 = v2h{sp[1], sp[1]};
  h.v[0] = dequant8(f.q.x, s0);
  h.v[1] = dequant8(f.q.y, s0);
  h.v[2] = dequant8(f.q.z, s1);
  h.v[3] = dequant8(f.q.w, s1);
}
// One of the four 8-element MFMA operands of a fragment.
__device__ inline v8h expand_part(const Frag4& f, int j) {
  const v2h sp = sig_pair(f.sc);
  const v2h sg = j < 2 ? v2h{sp[0], sp[0]} : v2h{sp[1], sp[1]};
  const uint32_t w = j == 0 ? f.q.x : j == 1 ? f.q.y : j == 2 ? f.q.z : f.q.w;
  return dequant8(w, sg);
}

// Work of one k step for one wave: MS row subtiles x NCG column groups.
// The MFMAs are ordered so consecutive ones update different accumulators.
template <int FMT, int MS, int NCG, typename Frag>
__device__ inline void step_compute(const Frag* fa, const Frag* fb, v4f (*acc)[NCG]) {
  if constexpr (FMT == 2) {
#pragma unroll
    for (int i = 0; i < MS; i++)
#pragma unroll
      for (int c = 0; c < NCG; c++) acc[i][c] = mma(fa[i], fb[c], acc[i][c]);
  } else {
    Half4 ha[MS];
#pragma unroll
    for (int i = 0; i < MS; i++) expand(fa[i], ha[i]);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int c = 0; c < NCG; c++) {
        const v8h hb = expand_part(fb[c], j);
#pragma unroll
        for (int i = 0; i < MS; i++)
          acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[i].v[j], hb, acc[i][c], 0, 0, 0);
      }
  }
}

// STAGE 0: gate/up (A = x codes gathered by token, B = w13, out = h [P][F]).
//   Workgroup tile: 64 rows of w13 (32 gate rows and the matching 32 up rows).
//   The 4 waves split K four ways (KS = 4, NS = 1).
// STAGE 1: down (A = h codes in sorted order, B = w2, out = y [P][H]).
//   Workgroup tile: 64 rows of w2.  Waves split K two ways and the 64 rows
//   two ways (KS = 2, NS = 2).
// NST > 0: every wave runs exactly NST k steps (K = 128 * NST * KS), fully
// unrolled with no branch in the step sequence; NST == 0: any K, runtime
// trip counts.
// LDS of one tile: the K-split partial tiles, the tile's token (gate/up) or
// row (down) indices and the NVFP4 activation row scales (read once, not per
// output).
template <int STAGE, int MS>
struct TileLds {
  static constexpr int KS = STAGE == 0 ? 4 : 2, TM = 16 * MS;
  float red[KS][TM][64 + 1];
  int tok[TM];
  float rgs[TM];
};

// Output store.  COH: a device-scope store, written through to the point
// where every XCD's loads meet (no L2 write-back is needed before another
// XCD reads it once a device-scope flag says it is there).
template <bool COH, typename T>
__device__ inline void st(T* p, T v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// One work-list entry `tile` x one 64-row weight slice `bx` (valid entry:
// tile < *a.ntiles).  Every thread of the 256-thread workgroup calls it
// (tid: its thread index); it contains workgroup barriers and leaves the LDS
// free only after the caller's next barrier.  COH: outputs stored with st<true>.
template <int FMT, int STAGE, int MS, int PF, int NST, bool PACKED, bool COH = false>
__device__ __forceinline__ void expert_tile(const GemmArgs& a, int tile, int bx, TileLds<STAGE, MS>& sm,
                                            int tid) {
  constexpr int KS = STAGE == 0 ? 4 : 2, NS = 4 / KS;
  constexpr int TM = 16 * MS, BN = 64, NCG = 4 / NS;
  typedef typename std::conditional<FMT == 2, Frag8, Frag4>::type Frag;
  auto& red = sm.red;
  int* tok = sm.tok;
  float* rgs = sm.rgs;

  const int el = a.worklist[2 * tile], m0 = a.worklist[2 * tile + 1];
  const int row0 = a.offsets[el] + m0;
  const int rows = min(TM, a.offsets[el + 1] - row0);

  const int wave = tid >> 6, lane = tid & 63;
  const int kpart = wave % KS, npart = wave / KS;
  const int r = lane & 15, g = lane >> 4;
  const int K = STAGE == 0 ? a.H : a.F;
  const int NW = STAGE == 0 ? 2 * a.F : a.H;              // rows of the weight matrix
  const int row_bytes = FMT == 2 ? K : K / 2;
  const int sc_bytes = FMT == 2 ? K / 32 : K / 16;
  const uint8_t* wexp = a.w_codes + (size_t)el * NW * row_bytes;
  const uint8_t* wsexp = a.w_sc + (size_t)el * NW * sc_bytes;

  // weight rows of this lane (column groups of 16 output columns)
  const uint8_t* brow[NCG];
  const uint8_t* bsrow[NCG];
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int cg = npart * NCG + c;   // 0..3 within the 64-row tile
    int n;
    if (STAGE == 0)   // column groups 0,1: gate rows; 2,3: the matching up rows
      n = (cg < 2 ? 0 : a.F) + bx * 32 + 16 * (cg & 1) + r;
    else
      n = bx * BN + 16 * cg + r;
    if (PACKED) {   // the row group's first tile (all K steps of a group are contiguous)
      const size_t tiles = (size_t)((n - r) / 16) * (K / 128);
      brow[c] = wexp + tiles * (FMT == 2 ? 2048 : 1024);
      bsrow[c] = wsexp + tiles * (FMT == 2 ? 64 : 128);
    } else {
      brow[c] = wexp + (size_t)n * row_bytes;
      bsrow[c] = wsexp + (size_t)n * sc_bytes;
    }
  }

  if (tid < TM) {
    const int m = tid;
    const int tk = m < rows ? (STAGE == 0 ? a.sorted[row0 + m] / a.k : row0 + m) : -1;
    tok[m] = tk;
    if (FMT == 1) rgs[m] = tk >= 0 ? a.a_gs[tk] : 0.0f;
  }
  __syncthreads();

  // activation rows of this lane; rows past the tile read the tile's first
  // row (MFMA rows are independent, their outputs are discarded)
  const uint8_t* arow[MS];
  const uint8_t* asrow[MS];
#pragma unroll
  for (int i = 0; i < MS; i++) {
    const int t = tok[16 * i + r];
    const int tt = t >= 0 ? t : tok[0];
    arow[i] = a.a_codes + (size_t)tt * row_bytes;
    asrow[i] = a.a_sc + (size_t)tt * sc_bytes;
  }

  v4f acc[MS][NCG];
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int c = 0; c < NCG; c++) acc[i][c] = v4f{0, 0, 0, 0};

  // Ring of PF k steps in flight.  No load sits under a branch: a divergent
  // or conditional load makes the compiler drain every outstanding load at
  // the join, which serializes the pipeline.
  Frag fa[PF][MS], fb[PF][NCG];
  auto issue = [&](int step, Frag* A, Frag* B) {
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      if (PACKED) load_frag_packed(B[c], brow[c], bsrow[c], step, lane);
      else load_frag<true>(B[c], brow[c], bsrow[c], step * 128, g);
    }
#pragma unroll
    for (int i = 0; i < MS; i++) load_frag(A[i], arow[i], asrow[i], step * 128, g);
  };
  if constexpr (NST > 0) {
    const int s0 = kpart * NST;
#pragma unroll
    for (int j = 0; j < PF && j < NST; j++) issue(s0 + j, fa[j], fb[j]);
#pragma unroll
    for (int s = 0; s < NST; s++) {
      // a wave whose operands have arrived issues ahead of the others
      // (MXFP8 decode gate/up 557 -> 544 us on one box)
      __builtin_amdgcn_s_setprio(1);
      step_compute<FMT, MS, NCG>(fa[s % PF], fb[s % PF], acc);
      __builtin_amdgcn_s_setprio(0);
      if (s + PF < NST) issue(s0 + s + PF, fa[s % PF], fb[s % PF]);
    }
  } else {
    const int nsteps = K / 128;
    const int s0 = kpart * nsteps / KS, s1 = (kpart + 1) * nsteps / KS;
    const int slast = s1 - 1;
    if (s0 < s1) {
#pragma unroll
      for (int j = 0; j < PF; j++) issue(min(s0 + j, slast), fa[j], fb[j]);
    }
    // steps past the wave's range re-read its last step (a cache hit)
    for (int s = s0; s < s1; s += PF) {
#pragma unroll
      for (int j = 0; j < PF; j++) {
        if (s + j < s1) step_compute<FMT, MS, NCG>(fa[j], fb[j], acc);
        issue(min(s + j + PF, slast), fa[j], fb[j]);
      }
    }
  }

  // partial tiles -> LDS (acc reg q of lane l is D[4*(l/16)+q][l%16])
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int c = 0; c < NCG; c++)
#pragma unroll
      for (int q = 0; q < 4; q++) red[kpart][16 * i + 4 * g + q][16 * (npart * NCG + c) + r] = acc[i][c][q];
  __syncthreads();

  auto ksum = [&](int m, int c) {
    float v = red[0][m][c];
#pragma unroll
    for (int p = 1; p < KS; p++) v += red[p][m][c];
    return v;
  };
  if (STAGE == 0) {
    // 32 consecutive threads hold one row's 32 h columns; for MXFP8 they are
    // one scale block, encoded here (amax over the 32 lanes, then each lane
    // its code).  Every thread runs every iteration (TM * 32 is a multiple of
    // 256), so the lane exchanges always see all 32 lanes.
    const float inv_c = 1.0f / a.cap;
    for (int idx = tid; idx < TM * 32; idx += 256) {
      const int m = idx >> 5, c = idx & 31;
      const bool live = m < rows;
      float gv = ksum(m, c), uv = ksum(m, 32 + c);
      if (FMT == 1) {
        const ScalePair ga = split_scale(rgs[m]);
        gv = apply_scale(gv, ga * split_scale(a.w_gs[3 * el + 0]));
        uv = apply_scale(uv, ga * split_scale(a.w_gs[3 * el + 1]));
      }
      const float h = cap_swiglu(gv, uv, a.cap_form, a.cap, inv_c);
      if (FMT == 2) {
        float am = live ? fabsf(h) : 0.0f;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
        const int E = mx_exponent(am);
        const uint32_t code = mx_encode(h, pow2f(-E));
        if (live) {
          st<COH>(a.out_q + (size_t)(row0 + m) * a.F + bx * 32 + c, (uint8_t)code);
          if (c == 0) st<COH>(a.out_s + (size_t)(row0 + m) * (a.F / 32) + bx, (uint8_t)(E + 127));
        }
      } else if (live) {
        st<COH>(a.out + (size_t)(row0 + m) * a.F + bx * 32 + c, h);
      }
    }
  } else {
    for (int idx = tid; idx < TM * BN; idx += 256) {
      const int m = idx >> 6, c = idx & 63;
      if (m >= rows) continue;
      float yv = ksum(m, c);
      if (FMT == 1) yv = apply_scale(yv, split_scale(rgs[m]) * split_scale(a.w_gs[3 * el + 2]));
      st<COH>(a.out + (size_t)(row0 + m) * a.H + bx * BN + c, yv);
    }
  }
}


}  // namespace moe
