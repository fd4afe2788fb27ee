// Grouped expert GEMMs on gfx950 MFMA (the two expert GEMMs of the SGLang
// cookbook's MegaMoE description, section 2; W4A4 / W8A8 per Miles docs
// section 5.3; the expert layout of the NVFP4 / MXFP8 checkpoint, SGLang
// cookbook section 2 "Checkpoints").
//
// Work: the dispatch work list holds one entry per (local expert, block of
// TM = 16*MS sorted rows); grid.y walks it (entries past the device-side
// count exit at once), grid.x walks 64-row slices of the expert's weight
// matrix.  Each workgroup's 4 waves split K four ways; every wave loads its
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
//   operand, and E2M1 times an E4M3 scale needs up to 7 significant bits, so
//   both operands are expanded in registers to f16 = E2M1 value * block
//   scale (exact: at most 7 bits, magnitudes 2^-10 .. 2688) and multiplied
//   on v_mfma_f32_16x16x32_f16 (products exact in the fp32 accumulator).
//   The two fp32 tensor/row scales are applied in the epilogue.  Each lane
//   loads 16 bytes = 32 consecutive E2M1 codes per 128-wide k step and feeds
//   8 of them to each of four MFMAs; both operands use the same k mapping.
#include <type_traits>

#include "moe_common.h"
#include "launch.h"

namespace moe {

// E2M1 x 8 (one 32-bit word, low nibble first) -> f16 x 8 scaled by sig.
__device__ inline v8h dequant8(uint32_t word, v2h sig2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sig2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sig2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sig2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sig2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ inline v2h e4m3_to_h2(uint32_t c) {
  const _Float16 s = (_Float16)e4m3_decode(c);
  return v2h{s, s};
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

__device__ inline void load_frag(Frag8& f, const uint8_t* row, const uint8_t* sc_row, int k0, int g) {
  f.lo = *reinterpret_cast<const uint4*>(row + k0 + 16 * g);
  f.hi = *reinterpret_cast<const uint4*>(row + k0 + 64 + 16 * g);
  f.sc = sc_row[k0 / 32 + g];
}
__device__ inline void load_frag(Frag4& f, const uint8_t* row, const uint8_t* sc_row, int k0, int g) {
  f.q = *reinterpret_cast<const uint4*>(row + k0 / 2 + 16 * g);
  const uint8_t* s = sc_row + k0 / 16 + 2 * g;
  f.sc = (uint32_t)s[0] | ((uint32_t)s[1] << 8);
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

// NVFP4: expand both fragments and issue four f16 MFMAs.
struct Half4 {
  v8h v[4];
};
__device__ inline void expand(const Frag4& f, Half4& h) {
  const v2h s0 = e4m3_to_h2(f.sc & 0xFF), s1 = e4m3_to_h2(f.sc >> 8);
  h.v[0] = dequant8(f.q.x, s0);
  h.v[1] = dequant8(f.q.y, s0);
  h.v[2] = dequant8(f.q.z, s1);
  h.v[3] = dequant8(f.q.w, s1);
}
__device__ inline v4f mma(const Half4& a, const Half4& b, v4f c) {
#pragma unroll
  for (int j = 0; j < 4; j++) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// STAGE 0: gate/up (A = x codes gathered by token, B = w13, out = h [P][F]).
// STAGE 1: down (A = h codes in sorted order, B = w2, out = y [P][H]).
template <int FMT, int STAGE, int MS>
__global__ __launch_bounds__(256) void k_expert_gemm(GemmArgs a) {
  constexpr int TM = 16 * MS, BN = 64, NCG = 4;
  typedef typename std::conditional<FMT == 2, Frag8, Frag4>::type Frag;
  __shared__ float red[4][TM][BN + 1];
  __shared__ int tok[TM];

  const int tile = blockIdx.y;
  if (tile >= a.ntiles[0]) return;
  const int el = a.worklist[2 * tile], m0 = a.worklist[2 * tile + 1];
  const int row0 = a.offsets[el] + m0;
  const int rows = min(TM, a.offsets[el + 1] - row0);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = STAGE == 0 ? a.H : a.F;
  const int NW = STAGE == 0 ? 2 * a.F : a.H;              // rows of the weight matrix
  const int row_bytes = FMT == 2 ? K : K / 2;
  const int sc_bytes = FMT == 2 ? K / 32 : K / 16;
  const uint8_t* wexp = a.w_codes + (size_t)el * NW * row_bytes;
  const uint8_t* wsexp = a.w_sc + (size_t)el * NW * sc_bytes;

  if (threadIdx.x < TM) {
    const int m = threadIdx.x;
    tok[m] = m < rows ? (STAGE == 0 ? a.sorted[row0 + m] / a.k : row0 + m) : -1;
  }
  __syncthreads();

  // rows of this lane's operands
  const uint8_t* arow[MS];
  const uint8_t* asrow[MS];
  bool avalid[MS];
#pragma unroll
  for (int i = 0; i < MS; i++) {
    const int t = tok[16 * i + r];
    avalid[i] = t >= 0;
    const int tt = t >= 0 ? t : 0;
    arow[i] = a.a_codes + (size_t)tt * row_bytes;
    asrow[i] = a.a_sc + (size_t)tt * sc_bytes;
  }
  const uint8_t* brow[NCG];
  const uint8_t* bsrow[NCG];
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    int n;
    if (STAGE == 0)   // column groups 0,1: gate rows; 2,3: the matching up rows
      n = (c < 2 ? 0 : a.F) + blockIdx.x * 32 + 16 * (c & 1) + r;
    else
      n = blockIdx.x * BN + 16 * c + r;
    brow[c] = wexp + (size_t)n * row_bytes;
    bsrow[c] = wsexp + (size_t)n * sc_bytes;
  }

  v4f acc[MS][NCG];
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int c = 0; c < NCG; c++) acc[i][c] = v4f{0, 0, 0, 0};

  const int nsteps = K / 128;
  const int s0 = wave * nsteps / 4, s1 = (wave + 1) * nsteps / 4;
  Frag fa[MS], fb[NCG];
  if (s0 < s1) {
#pragma unroll
    for (int c = 0; c < NCG; c++) load_frag(fb[c], brow[c], bsrow[c], s0 * 128, g);
#pragma unroll
    for (int i = 0; i < MS; i++) {
      if (avalid[i]) load_frag(fa[i], arow[i], asrow[i], s0 * 128, g);
      else zero_frag(fa[i]);
    }
  }
  for (int s = s0; s < s1; s++) {
    Frag na[MS], nb[NCG];
    const bool more = s + 1 < s1;
    if (more) {
#pragma unroll
      for (int c = 0; c < NCG; c++) load_frag(nb[c], brow[c], bsrow[c], (s + 1) * 128, g);
#pragma unroll
      for (int i = 0; i < MS; i++) {
        if (avalid[i]) load_frag(na[i], arow[i], asrow[i], (s + 1) * 128, g);
        else zero_frag(na[i]);
      }
    }
    if constexpr (FMT == 2) {
#pragma unroll
      for (int i = 0; i < MS; i++)
#pragma unroll
        for (int c = 0; c < NCG; c++) acc[i][c] = mma(fa[i], fb[c], acc[i][c]);
    } else {
      Half4 hb[NCG];
#pragma unroll
      for (int c = 0; c < NCG; c++) expand(fb[c], hb[c]);
#pragma unroll
      for (int i = 0; i < MS; i++) {
        Half4 ha;
        expand(fa[i], ha);
#pragma unroll
        for (int c = 0; c < NCG; c++) acc[i][c] = mma(ha, hb[c], acc[i][c]);
      }
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < NCG; c++) fb[c] = nb[c];
#pragma unroll
      for (int i = 0; i < MS; i++) fa[i] = na[i];
    }
  }

  // partial tiles -> LDS (acc reg q of lane l is D[4*(l/16)+q][l%16])
#pragma unroll
  for (int i = 0; i < MS; i++)
#pragma unroll
    for (int c = 0; c < NCG; c++)
#pragma unroll
      for (int q = 0; q < 4; q++) red[wave][16 * i + 4 * g + q][16 * c + r] = acc[i][c][q];
  __syncthreads();

  if (STAGE == 0) {
    const float inv_c = 1.0f / a.cap;
    for (int idx = threadIdx.x; idx < TM * 32; idx += 256) {
      const int m = idx >> 5, c = idx & 31;
      if (m >= rows) continue;
      float gv = ((red[0][m][c] + red[1][m][c]) + red[2][m][c]) + red[3][m][c];
      float uv = ((red[0][m][32 + c] + red[1][m][32 + c]) + red[2][m][32 + c]) + red[3][m][32 + c];
      if (FMT == 1) {
        const float ga = a.a_gs[tok[m]];
        gv = (gv * ga) * a.w_gs[3 * el + 0];
        uv = (uv * ga) * a.w_gs[3 * el + 1];
      }
      const float h = cap_swiglu(gv, uv, a.cap_form, a.cap, inv_c);
      a.out[(size_t)(row0 + m) * a.F + blockIdx.x * 32 + c] = h;
    }
  } else {
    for (int idx = threadIdx.x; idx < TM * BN; idx += 256) {
      const int m = idx >> 6, c = idx & 63;
      if (m >= rows) continue;
      float yv = ((red[0][m][c] + red[1][m][c]) + red[2][m][c]) + red[3][m][c];
      if (FMT == 1) yv = (yv * a.a_gs[row0 + m]) * a.w_gs[3 * el + 2];
      a.out[(size_t)(row0 + m) * a.H + blockIdx.x * BN + c] = yv;
    }
  }
}

int gemm_tile_m(int T, int k, int E_local) {
  // average rows per local expert; small batches use 32-row tiles
  const long pairs = (long)T * k;
  return pairs / (E_local > 0 ? E_local : 1) > 24 ? 64 : 32;
}

static int launch_any(const GemmArgs& a, int stage, hipStream_t stream) {
  const dim3 block(256);
  const dim3 grid(stage == 0 ? a.F / 32 : a.H / 64, a.max_tiles);
  const bool big = a.tile_m == 64;
#define MOE_LAUNCH(FMT, ST, MS) \
  hipLaunchKernelGGL((k_expert_gemm<FMT, ST, MS>), grid, block, 0, stream, a)
  if (a.fmt == 2) {
    if (stage == 0) { if (big) MOE_LAUNCH(2, 0, 4); else MOE_LAUNCH(2, 0, 2); }
    else            { if (big) MOE_LAUNCH(2, 1, 4); else MOE_LAUNCH(2, 1, 2); }
  } else {
    if (stage == 0) { if (big) MOE_LAUNCH(1, 0, 4); else MOE_LAUNCH(1, 0, 2); }
    else            { if (big) MOE_LAUNCH(1, 1, 4); else MOE_LAUNCH(1, 1, 2); }
  }
#undef MOE_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_gateup(const GemmArgs& a, hipStream_t stream) { return launch_any(a, 0, stream); }
int launch_gemm_down(const GemmArgs& a, hipStream_t stream) { return launch_any(a, 1, stream); }

}  // namespace moe
