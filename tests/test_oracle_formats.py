"""Pins of the oracle's element formats and block quantizers.

Each check ties the oracle to something other than itself: torch's float8
dtypes (a library), exhaustive exact-rational nearest-value search over every
bf16 input, exactly representable constructions, and the published range
invariants of the block formats.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _all_bf16_f32():
    v = F.bf16_bits_to_f32(ALL_BF16)
    return v[np.isfinite(v)]


# ---------------------------------------------------------------- tables ----

def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.e8m0_decode(codes), ref)


def test_e2m1_table_is_ocp_fp4():
    # OCP MX FP4 (E2M1) magnitudes
    assert list(F.E2M1_MAG) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.e2m1_decode(np.uint8(0xF)) == -6.0 and F.e2m1_decode(np.uint8(0x9)) == -0.5


# ------------------------------------------------------------ encoders -----

def test_e4m3_encode_all_bf16_matches_torch():
    v = _all_bf16_f32()
    got = F.e4m3_encode(v)
    inr = np.abs(v) <= 464.0          # torch saturates nothing: beyond 464 it gives NaN
    ref = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], ref)
    big = ~inr
    assert np.all((got[big] & 0x7F) == 0x7E)                     # satfinite
    assert np.array_equal((got[big] >> 7).astype(bool), np.signbit(v[big]))


def test_e4m3_encode_random_f32_matches_torch():
    g = np.random.default_rng(5)
    v = (g.standard_normal(200000) * np.exp(g.uniform(-25, 7, 200000))).astype(np.float32)
    v = v[np.abs(v) <= 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(v), ref)


def _nearest_exact(v: float, mags, sign_shift):
    """Exact-rational nearest value; ties to even code; satfinite; signed zero."""
    a = abs(Fraction(v))
    best, bestd = None, None
    for c, m in enumerate(mags):
        d = abs(a - Fraction(m))
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    if a >= Fraction(mags[-1]):
        best = len(mags) - 1
    sign = 1 if np.signbit(v) else 0
    return best | (sign << sign_shift)


def test_e2m1_encode_exhaustive_bf16():
    v = _all_bf16_f32()
    got = F.e2m1_encode(v)
    # all distinct magnitudes (the table is tiny): check every bf16 value exactly
    mags = [float(m) for m in F.E2M1_MAG]
    ref = np.array([_nearest_exact(float(x), mags, 3) for x in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e2m1_encode_midpoints_and_edges():
    # midpoints go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0,
    # 2.5->2.0, 3.5->4.0, 5.0->4.0; above 6 saturates; -0 keeps its sign
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 1e30, -0.0, -0.25, np.inf], dtype=np.float32)
    exp = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.0, -0.0, 6.0]
    got = F.e2m1_decode(F.e2m1_encode(v))
    assert list(got) == exp
    assert list(np.signbit(got)) == [False] * 9 + [True, True, False]
    assert F.e2m1_encode(np.float32(np.nan)) == 0


def test_e4m3_encode_sample_exact():
    g = np.random.default_rng(1)
    v = (g.standard_normal(3000) * np.exp(g.uniform(-12, 7, 3000))).astype(np.float32)
    mags = [float(m) for m in F.E4M3_MAG]
    ref = np.array([_nearest_exact(float(x), mags, 7) for x in v], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(v), ref)


# ---------------------------------------------------------------- bf16 -----

def test_bf16_round_matches_torch_on_f32():
    g = np.random.default_rng(2)
    v = (g.standard_normal(100000) * np.exp(g.uniform(-100, 87, 100000))).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, 3.39e38, -3.4e38, 1e-45, 1.1754944e-38], dtype=np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_round_f64(v.astype(np.float64)), ref)


def test_bf16_round_f64_single_rounding():
    # x = 1 + 2^-8 + 2^-30: a first rounding to fp32 would give 1 + 2^-8
    # (a bf16 tie that goes to 1.0); rounding once goes up to 1 + 2^-7.
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30), 1.0 + 2.0 ** -8])
    got = F.bf16_bits_to_f32(F.bf16_round_f64(x)).astype(np.float64)
    assert list(got) == [1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 1.0]


# -------------------------------------------------------------- packing ----

def test_nibble_order():
    assert F.pack_nibbles(np.array([[0x1, 0x2, 0xF, 0x0]], dtype=np.uint8)).tolist() == [[0x21, 0x0F]]
    g = np.random.default_rng(3)
    c = g.integers(0, 16, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)


# ------------------------------------------------------------- MXFP8 -------

def _rows(seed, R=64, K=256):
    g = np.random.default_rng(seed)
    mag = np.exp(g.uniform(-30, 30, size=(R, 1)))
    v = (g.standard_normal((R, K)) * mag).astype(np.float32)
    v[0] = 0.0
    v[1, :32] = 0.0
    v[2] = np.float32(1e-40)                # subnormal row
    v[3, 5] = -0.0
    v[4] *= np.float32(1e20)
    return v


def test_mxfp8_scale_invariants():
    v = _rows(10)
    codes, scales = F.quantize_mxfp8(v)
    assert scales.max() <= 254
    vals = F.e4m3_decode(codes).reshape(v.shape[0], -1, 32)
    blocks = v.reshape(v.shape[0], -1, 32)
    amax = np.abs(blocks).max(-1)
    bm = np.abs(vals).max(-1)
    nz = amax > 0
    unclamped = nz & (scales > 0)
    assert np.all((bm[unclamped] >= 256) & (bm[unclamped] <= 448))
    assert np.all(scales[~nz] == 0)
    assert np.all(np.abs(vals[~nz]) == 0)


def test_mxfp8_roundtrip_error_bound():
    v = _rows(11)
    codes, scales = F.quantize_mxfp8(v)
    d = F.dequantize_mxfp8(codes, scales)
    X = F.e8m0_decode(scales).repeat(32, axis=-1)
    y = v.astype(np.float64) / X                       # element on the E4M3 grid scale
    ay = np.abs(y)
    # half an E4M3 step: 2^(floor(log2|y|)-4) for normals, 2^-10 for subnormals
    e = np.floor(np.log2(np.maximum(ay, 2.0 ** -6)))
    half = np.where(ay < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    sat = ay > 448
    err = np.abs(d / X - y)
    assert np.all(err[~sat] <= half[~sat] * (1 + 1e-12))
    assert np.all(np.abs(d / X)[sat] == 448)
    assert np.array_equal(np.signbit(d), np.signbit(v))


def test_mxfp8_exactly_representable_is_lossless():
    g = np.random.default_rng(12)
    R, K = 16, 256
    nb = K // 32
    E = g.integers(-120, 100, size=(R, nb))
    codes = g.integers(0, 256, size=(R, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    # force each block's largest magnitude into [256, 448]
    blk = codes.reshape(R, nb, 32)
    blk[:, :, 0] = (blk[:, :, 0] & 0x80) | g.integers(0x78, 0x7F, size=(R, nb))
    blk[:, :, 1:] = np.where((blk[:, :, 1:] & 0x7F) > 0x7E, 0x00, blk[:, :, 1:])
    codes = blk.reshape(R, K)
    v = (F.e4m3_decode(codes).reshape(R, nb, 32) * np.ldexp(1.0, E)[..., None]).reshape(R, K).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), (F.e4m3_decode(codes).reshape(R, nb, 32) * np.ldexp(1.0, E)[..., None]).reshape(R, K))
    c2, s2 = F.quantize_mxfp8(v)
    assert np.array_equal(s2.astype(np.int64), E + 127)
    assert np.array_equal(c2, codes)


# ------------------------------------------------------------- NVFP4 -------

def test_nvfp4_exactly_representable_is_lossless():
    g = np.random.default_rng(13)
    R, K = 12, 256
    nb = K // 16
    gs0 = np.float32(2.0 ** g.integers(-20, 5))
    codes = g.integers(0, 16, size=(R, nb, 16)).astype(np.uint8)
    codes[:, :, 3] = 0x7 | (codes[:, :, 3] & 0x8)                  # a +-6 in every block
    sc = g.integers(0x08, 0x7F, size=(R, nb)).astype(np.uint8)       # normal E4M3 scales
    sc[:, 0] = 0x7E                                                  # the row maximum: 448
    v = (F.e2m1_decode(codes) * F.e4m3_decode(sc)[..., None] * np.float64(gs0)).reshape(R, K)
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)
    p, s, gs = F.quantize_nvfp4(v32, domain="row")
    assert np.all(gs == gs0)
    assert np.array_equal(s, sc)
    c = F.unpack_nibbles(p).reshape(R, nb, 16)
    mag = lambda x: x & 7  # noqa: E731
    assert np.array_equal(mag(c), mag(codes))
    nz = mag(codes) != 0
    assert np.array_equal((c & 8)[nz], (codes & 8)[nz])
    assert np.array_equal(F.dequantize_nvfp4(p, s, gs), v)


def test_nvfp4_scale_invariants():
    v = _rows(14, R=48, K=512)
    v = v[np.abs(v).max(1) < 1e36]             # keep rows whose scale math stays finite
    p, s, gs = F.quantize_nvfp4(v, domain="row")
    c = F.unpack_nibbles(p).reshape(v.shape[0], -1, 16)
    sig = F.e4m3_decode(s)
    A = np.abs(v).max(1)
    nz = A > 0
    # the block holding the row maximum gets the largest E4M3 scale
    imax = np.abs(v).argmax(1) // 16
    assert np.all(sig[nz, imax[nz]] == 448)
    # any block with a normal scale uses the full E2M1 range
    normal = sig >= 2.0 ** -6
    assert np.all((np.abs(F.e2m1_decode(c)).max(-1) == 6)[normal])
    assert np.all(gs[~nz] == 1.0) and np.all(s[~nz] == 0)


def test_nvfp4_roundtrip_error_bound():
    g = np.random.default_rng(15)
    v = (g.standard_normal((40, 4608)) * np.exp(g.uniform(-20, 20, (40, 1)))).astype(np.float32)
    p, s, gs = F.quantize_nvfp4(v, domain="row")
    d = F.dequantize_nvfp4(p, s, gs).reshape(40, -1, 16)
    unit = (F.e4m3_decode(s) * gs[:, None].astype(np.float64))[..., None]
    y = np.abs(v.reshape(40, -1, 16).astype(np.float64)) / unit
    # E2M1 half-steps: 0.25 below 2, 0.5 in [2,4), 1 in [4,6]; beyond 6 the
    # element saturates (the block scale rounded down by at most 1/16)
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    err = np.abs(np.abs(d) / unit - y)
    ok = (err <= half * (1 + 1e-6)) | ((y > 6) & (np.abs(d) / unit == 6) & (y < 6 * 1.0667))
    assert np.all(ok)


def test_nvfp4_tensor_domain_uses_one_scale():
    g = np.random.default_rng(16)
    v = (g.standard_normal((32, 64)) * 0.02).astype(np.float32)
    _, _, gs = F.quantize_nvfp4(v, domain="tensor")
    assert gs.shape == () and gs == np.float32(np.abs(v).max()) / np.float32(2688.0)
    p_row, _, gs_row = F.quantize_nvfp4(v, domain="row")
    assert gs_row.shape == (32,)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_quantizers_are_row_independent(fmt):
    g = np.random.default_rng(17)
    a = g.standard_normal((6, 512)).astype(np.float32)
    b = a.copy()
    b[1:] = g.standard_normal((5, 512)).astype(np.float32) * 100
    qa = F.quantize_mxfp8(a) if fmt == "mxfp8" else F.quantize_nvfp4(a)
    qb = F.quantize_mxfp8(b) if fmt == "mxfp8" else F.quantize_nvfp4(b)
    for x, y in zip(qa, qb):
        assert np.array_equal(np.asarray(x)[0], np.asarray(y)[0])
