// One-time repack of expert weights into the packed layout (tiles of 16
// rows x 128 columns stored in MFMA-operand lane order; include/moe.h,
// moe_prepare_weights).  Pure byte permutation: the gather of every 16-byte
// code chunk and scale byte from the canonical row-major arrays.  Runs once
// at load time; HBM-bound.
#include "moe_common.h"
#include "launch.h"

namespace moe {

// One thread per (tile, lane).  fmt 1 NVFP4, 2 MXFP8.  N rows, K columns,
// nmat matrices of that shape back to back (the local experts).
__global__ __launch_bounds__(256) void k_pack(int fmt, const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, long nmat, int N, int K,
                                              uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int NS = K / 128, NG = N / 16;
  const long tiles = nmat * NG * NS;
  if (idx >= tiles * 64) return;
  const int l = (int)(idx & 63);
  const long tile = idx >> 6;                  // (mat, g, s)
  const int s = (int)(tile % NS);
  const long mg = tile / NS;                   // mat * NG + g
  const long row = mg * 16 + (l & 15);         // global row over all matrices
  const int grp = l >> 4;
  if (fmt == 1) {
    const long rb = K / 2, sb = K / 16;
    const uint4 q = *reinterpret_cast<const uint4*>(codes + row * rb + s * 64 + 16 * grp);
    *reinterpret_cast<uint4*>(pcodes + tile * 1024 + 16 * l) = q;
    const uint8_t* sc = scales + row * sb + s * 8 + 2 * grp;
    pscales[tile * 128 + 2 * l] = sc[0];
    pscales[tile * 128 + 2 * l + 1] = sc[1];
  } else {
    const long rb = K, sb = K / 32;
    const uint8_t* src = codes + row * rb + s * 128 + 16 * grp;
    *reinterpret_cast<uint4*>(pcodes + tile * 2048 + 16 * l) = *reinterpret_cast<const uint4*>(src);
    *reinterpret_cast<uint4*>(pcodes + tile * 2048 + 1024 + 16 * l) = *reinterpret_cast<const uint4*>(src + 64);
    pscales[tile * 64 + l] = scales[row * sb + s * 4 + grp];
  }
}

int launch_pack(int fmt, const uint8_t* codes, const uint8_t* scales, long nmat, int N, int K,
                uint8_t* pcodes, uint8_t* pscales, hipStream_t stream) {
  const long threads = nmat * (N / 16) * (K / 128) * 64;
  if (threads <= 0) return 0;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, fmt, codes, scales,
                     nmat, N, K, pcodes, pscales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
