"""Element formats and block quantizers (oracle side, test infrastructure only).

The pages name the formats only as "NVFP4" and "MXFP8" (SGLang cookbook,
section 2 "Checkpoints"; TokenSpeed blog, "What's new" table, Checkpoint
row).  The definitions below are the public conventions those names refer to:

* E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6.  Code = sign<<3 | exponent<<1 | mantissa.
* E4M3 (FP8, "FN" variant): bias 7, subnormals m*2^-9, largest finite 448;
  0x7F / 0xFF are NaN and never produced here.
* E8M0: unsigned power of two 2^(c-127) for c = 0..254; 255 (NaN) never
  produced.

Readings where the pages are silent (numbered R1, R2, ... throughout this package):

* R3 (MX scale): X = 2^(floor(log2 amax) - 8), 8 being the E4M3 emax; the
  exponent is clamped to [-127, 127]; elements saturate to +-448.
* R4 (rounding): round to nearest, ties to the even code (the code whose
  least significant bit is 0), saturate to the largest finite magnitude,
  keep the sign of zero.  A NaN operand (only reachable as 0*inf inside a
  degenerate NVFP4 block whose scale product underflows) encodes as +0.
* R1/R2 (NVFP4 fp32 scale): per row of an activation matrix (the scale must
  cover the expert's whole input width, SGLang cookbook section 2
  "Parallelism"), per whole (expert, matrix) tensor for weights.  Two
  alternatives for activations are kept selectable: one scale for the whole
  activation tensor of a call ("tensor"), or a fixed scale ("static").
  gs = amax / 2688 (2688 = 6 * 448); block scale s = E4M3(a_b / (6*gs));
  reciprocal r = 1 / (s*gs); codes E2M1(v * r).  Every step is one IEEE fp32
  operation (division, then multiplication), never fused.
* R5 (packing): element 2i in the low nibble of byte i, element 2i+1 in the
  high nibble.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Value tables, built from the field definitions above.
# --------------------------------------------------------------------------


def _e2m1_table() -> np.ndarray:
    mags = []
    for c in range(8):
        e, m = c >> 1, c & 1
        mags.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0))
    return np.array(mags, dtype=np.float64)


def _e4m3_table() -> np.ndarray:
    mags = []
    for c in range(0x7F):  # 0x7F is NaN
        e, m = c >> 3, c & 7
        mags.append(m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0))
    return np.array(mags, dtype=np.float64)


E2M1_MAG = _e2m1_table()   # index = 3-bit magnitude code, increasing
E4M3_MAG = _e4m3_table()   # index = 7-bit magnitude code, increasing


def _encode_nearest(v: np.ndarray, mags: np.ndarray, sign_shift: int) -> np.ndarray:
    """Nearest entry of the increasing magnitude table ``mags``.

    Ties pick the even magnitude code; magnitudes above the table saturate to
    its last entry; the sign bit (bit ``sign_shift``) copies the sign of v,
    including for zero.  NaN encodes as +0.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    top = len(mags) - 1
    hi = np.searchsorted(mags, a, side="left")          # first mags[hi] >= a
    hi = np.minimum(hi, top)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]                                   # exact (see tests)
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= mags[top], top, code)            # saturate
    sign = np.signbit(v) & ~nan
    return (code | (sign.astype(np.int64) << sign_shift)).astype(np.uint8)


def e2m1_encode(v) -> np.ndarray:
    """fp32 values -> E2M1 codes (uint8, low 4 bits used)."""
    return _encode_nearest(v, E2M1_MAG, 3)


def e2m1_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """fp32 values -> E4M3 codes (uint8), satfinite."""
    return _encode_nearest(v, E4M3_MAG, 7)


def e4m3_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    mag = E4M3_MAG[np.minimum(c & 0x7F, 0x7E)]
    return np.where(c & 0x80, -mag, mag)


def e8m0_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    return np.ldexp(1.0, c - 127)


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returning
    the bf16 bit patterns as uint16.  Rounds once, directly from float64.
    Magnitudes beyond the largest finite bf16 become +-inf (RNE overflow)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)              # 8 significant bits; subnormal floor
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    r = np.where(x == 0, x, r)               # keeps the sign of zero
    big = np.abs(r) > 3.3895313892515355e38  # (2 - 2^-7) * 2^127
    r = np.where(big, np.copysign(np.inf, x), r)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Nibble packing (reading R5)
# --------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# MXFP8: E4M3 elements, one E8M0 scale per 32 consecutive elements of a row.
# --------------------------------------------------------------------------

MX_BLOCK = 32
NV_BLOCK = 16


def quantize_mxfp8(v: np.ndarray):
    """Quantize fp32 rows [..., K] (K % 32 == 0) to MXFP8.

    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float32)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)                         # fp32
    _, ex = np.frexp(amax.astype(np.float64))                       # amax = m*2^ex
    e = ex - 1                                                      # floor(log2 amax)
    E = np.clip(e - 8, -127, 127)
    E = np.where(amax == 0, -127, E)                                # scale code 0
    step = np.ldexp(np.float32(1.0), -E).astype(np.float32)         # 2^-E, exact fp32
    scaled = blocks * step[..., None]                               # fp32, exact
    codes = e4m3_encode(scaled).reshape(v.shape)
    scales = (E + 127).astype(np.uint8)
    return codes, scales


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    """MXFP8 -> float64 values (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


# --------------------------------------------------------------------------
# NVFP4: E2M1 elements, one E4M3 scale per 16 consecutive elements of a row,
# one fp32 scale per scale domain (a row for activations, a whole tensor for
# weights).
# --------------------------------------------------------------------------

_F32 = np.float32


def _nvfp4_blocks(blocks: np.ndarray, gs: np.ndarray):
    """blocks: fp32 [..., nb, 16]; gs: fp32 [...] broadcastable to blocks[..., 0, 0].
    Returns codes uint8 [..., nb, 16] and block-scale codes uint8 [..., nb]."""
    a_b = np.max(np.abs(blocks), axis=-1)                           # fp32
    denom = (_F32(6.0) * gs).astype(_F32)                          # rounded product
    s_f = (a_b / denom[..., None]).astype(_F32)                    # fp32 division
    sc = e4m3_encode(s_f)
    sigma = e4m3_decode(sc).astype(_F32)
    t = (sigma * gs[..., None]).astype(_F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = (_F32(1.0) / t).astype(_F32)
        q = (blocks * r[..., None]).astype(_F32)
    codes = e2m1_encode(q)
    codes = np.where((sigma == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, sc


def nvfp4_global_scale(amax) -> np.ndarray:
    """fp32 scale of an NVFP4 scale domain with maximum magnitude amax:
    amax / 2688 as one IEEE fp32 division (2688 = 6 * 448, the largest E2M1
    value times the largest E4M3 value), and 1.0 for an all-zero domain."""
    A = np.asarray(amax, dtype=_F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(A == 0, _F32(1.0), (A / _F32(2688.0)).astype(_F32)).astype(_F32)


def quantize_nvfp4(v: np.ndarray, domain: str = "row", gs=None):
    """Quantize fp32 rows [R, K] (K % 16 == 0) to NVFP4.

    domain="row": one fp32 scale per row (activations, reading R1).
    domain="tensor": one fp32 scale for the whole array (weights, R2; the
        per-tensor alternative of R1 for activations).
    domain="static": the given fp32 scale `gs` for every row (the static
        alternative of R1: a scale fixed ahead of time, not taken from the
        data; block scales and codes saturate where the data exceed it).

    Row and tensor domains whose maximum is 0 take gs = 1 and all-zero codes
    and scales.  Returns (packed codes uint8 [R, K/2], scales uint8 [R, K/16],
    gs fp32 [R] for "row" or a 0-d fp32 array for "tensor" / "static").
    """
    v = np.asarray(v, dtype=np.float32)
    assert v.ndim == 2 and v.shape[1] % NV_BLOCK == 0
    R, K = v.shape
    if domain == "row":
        A = np.max(np.abs(v), axis=1).astype(_F32)                  # fp32 [R]
    elif domain == "tensor":
        A = np.max(np.abs(v)).reshape(()).astype(_F32) if v.size else np.zeros((), _F32)
    elif domain == "static":
        if gs is None or not (np.float32(gs) > 0 and np.isfinite(np.float32(gs))):
            raise ValueError("a static NVFP4 scale must be a positive finite fp32 value")
        A = None
    else:
        raise ValueError(domain)
    if A is not None:
        gs = nvfp4_global_scale(A)
        zero = np.broadcast_to(A == 0, (R,))
    else:
        gs = np.asarray(gs, dtype=_F32).reshape(())
        zero = np.zeros(R, dtype=bool)
    blocks = v.reshape(R, K // NV_BLOCK, NV_BLOCK)
    gs_rows = np.broadcast_to(gs, (R,)) if gs.ndim == 0 else gs
    codes, sc = _nvfp4_blocks(blocks, gs_rows)
    codes = np.where(zero[:, None, None], np.uint8(0), codes)
    sc = np.where(zero[:, None], np.uint8(0), sc).astype(np.uint8)
    return pack_nibbles(codes.reshape(R, K)), sc, gs


def dequantize_nvfp4(packed, scales, gs) -> np.ndarray:
    """NVFP4 -> float64 values, code * block scale * fp32 scale (exact in
    float64: at most 6 + 24 significant bits)."""
    codes = unpack_nibbles(packed)
    R, K = codes.shape
    vals = e2m1_decode(codes).reshape(R, K // NV_BLOCK, NV_BLOCK)
    sig = e4m3_decode(scales)[..., None]
    g = np.asarray(gs, dtype=np.float64)
    g = g.reshape(-1, 1, 1) if g.ndim == 1 else g
    return (vals * sig * g).reshape(R, K)
