"""Seeded synthetic inputs for the routed-expert MoE layer.

Shared by the tests, the benchmark and the smoke check.  This module only
draws random numbers and lays them out; it holds none of the layer's
arithmetic (no quantization, routing or matmul).  Every array is a pure
function of (seed, stream, ...) through numpy's PCG64 with a SeedSequence, so
any single expert can be regenerated on its own.

Streams: 0 = tokens x, 1 = router weight, 2 = router bias, (3, e) = float
weights of expert e, (4, e) = direct-code weights of expert e, (5, e) =
edge-case direct-code weights of expert e.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# The five workloads.  Shapes follow the Inkling 2 Small layer: hidden 4608,
# 384 experts, top-8, expert FFN 2304 (TokenSpeed blog "What's new" table;
# Miles docs section 2).


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    tokens: int
    hidden: int
    experts: int
    top_k: int
    ffn: int
    fmt: str                 # "nvfp4" | "mxfp8"
    seed: int
    bias: str = "normal"     # "normal" (N(0, 0.1)) | "zipf"
    expert_begin: int = 0
    num_local: int | None = None
    weights: str = "direct"  # "gaussian" (fp32 N(0, 0.02), encoded by the caller) | "direct"
    cap: float = 7.0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", "tiny MXFP8 layer: 16 tok, H256, E16 top-2, F128", 16, 256, 16, 2, 128, "mxfp8", 0,
                     weights="gaussian"),
    "decode_nvfp4": Workload("decode_nvfp4", "NVFP4 decode: 64 tok, H4608, E384 top-8, F2304",
                             64, 4608, 384, 8, 2304, "nvfp4", 1),
    "decode_mxfp8": Workload("decode_mxfp8", "MXFP8 decode: 192 tok, H4608, E384 top-8, F2304",
                             192, 4608, 384, 8, 2304, "mxfp8", 2),
    "prefill_nvfp4": Workload("prefill_nvfp4", "NVFP4 prefill: 16384 tok, H4608, E384 top-8, F2304, Zipf bias",
                              16384, 4608, 384, 8, 2304, "nvfp4", 3, bias="zipf"),
    "ep8_mxfp8": Workload("ep8_mxfp8", "EP8 share, MXFP8: 4096 tok, 48 local of 384 experts, H4608, F2304",
                          4096, 4608, 384, 8, 2304, "mxfp8", 4, num_local=48),
}

ZIPF_S = 1.1
ZIPF_LAMBDA = 0.05


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def tokens(seed: int, T: int, H: int) -> np.ndarray:
    """x ~ N(0, 1), as bf16 bits uint16 [T, H]."""
    return to_bf16_bits(rng(seed, 0).standard_normal((T, H), dtype=np.float32))


def router_weight(seed: int, E: int, H: int, sigma: float = 0.02) -> np.ndarray:
    """W_r ~ N(0, sigma^2), bf16 bits uint16 [E, H]."""
    return to_bf16_bits(rng(seed, 1).standard_normal((E, H), dtype=np.float32) * np.float32(sigma))


def router_bias(seed: int, E: int, kind: str = "normal") -> np.ndarray:
    """Selection bias fp32 [E].  "normal": N(0, 0.1).  "zipf": a Zipf(s=1.1)
    popularity over a random ranking of the experts, b = lambda*(ln p - mean
    ln p) with lambda = 0.05, which skews the expert load."""
    g = rng(seed, 2)
    if kind == "normal":
        return (g.standard_normal(E) * 0.1).astype(np.float32)
    if kind == "zipf":
        rank = g.permutation(E) + 1
        lp = -ZIPF_S * np.log(rank.astype(np.float64))
        lp = lp - np.log(np.exp(lp).sum())
        return (ZIPF_LAMBDA * (lp - lp.mean())).astype(np.float32)
    raise ValueError(kind)


def expert_float_weights(seed: int, e: int, H: int, Fd: int, sigma: float = 0.02):
    """Float weights of expert e: gate [F,H], up [F,H], down [H,F], N(0, sigma^2)."""
    g = rng(seed, 3, e)
    s = np.float32(sigma)
    gate = g.standard_normal((Fd, H), dtype=np.float32) * s
    up = g.standard_normal((Fd, H), dtype=np.float32) * s
    down = g.standard_normal((H, Fd), dtype=np.float32) * s
    return gate, up, down


# Direct-code weights: random valid encodings drawn straight from random
# bytes (no quantizer involved), sized so that an element's RMS is about
# 0.02 like the float recipe.  Used where encoding hundreds of full-size
# experts from floats would take minutes.  With b a uniform random byte:
#   NVFP4: code bytes = b (every nibble uniform over the 16 E2M1 codes);
#          block-scale bytes 0x68 + (b & 0xF) (E4M3 64 .. 240); fp32 scale
#          per matrix 2^-14 * U(0.9, 1.1).
#   MXFP8: E4M3 bytes (b & 0x80) | min(0x50 | (b & 0x2F), 0x7E): random sign,
#          exponent field in {10, 11, 14, 15}, any mantissa, never NaN;
#          E8M0 scale bytes 112 + bit0(b) + bit1(b) (2^-15 .. 2^-13).


def _bytes(g: np.random.Generator, shape) -> np.ndarray:
    return np.frombuffer(g.bytes(int(np.prod(shape))), dtype=np.uint8).reshape(shape)


def _mx_bytes(g: np.random.Generator, shape) -> np.ndarray:
    b = _bytes(g, shape)
    return (b & np.uint8(0x80)) | np.minimum(np.uint8(0x50) | (b & np.uint8(0x2F)), np.uint8(0x7E))


def _mx_scales(g: np.random.Generator, shape, shift: int) -> np.ndarray:
    b = _bytes(g, shape)
    return (np.uint8(112 + shift) + (b & np.uint8(1)) + ((b >> np.uint8(1)) & np.uint8(1))).astype(np.uint8)


def _nv_scales(g: np.random.Generator, shape) -> np.ndarray:
    return np.uint8(0x68) + (_bytes(g, shape) & np.uint8(0xF))


# Edge-case direct codes (edge=True, stream (5, e)): scale and element codes
# at the ends of their ranges, by expert e % 3:
#   NVFP4  0: every block scale subnormal (E4M3 0x01..0x07) or, one in ten,
#             zero; fp32 scales 2^-1 * U(0.9, 1.1) to keep the magnitudes
#          1: block scales over every normal E4M3 exponent (0x08..0x7E), one
#             in ten zero; fp32 scales 2^-20 * U(0.9, 1.1)
#          2: the plain draw above, but one block scale in ten zero
#   MXFP8  0: every element subnormal (exponent field 0) or zero, E8M0
#             scales 2^-6 .. 2^-4
#          1: elements over every exponent field, one in ten +-0, two in ten
#             subnormal; E8M0 scales 2^-27 .. 2^-1
#          2: the plain draw, one element in ten +-0


def _edge_codes(g: np.random.Generator, e: int, H: int, Fd: int, fmt: str, gain: float) -> dict:
    kind = e % 3
    if fmt == "nvfp4":
        def scales(shape):
            b, c = _bytes(g, shape), _bytes(g, shape)
            if kind == 0:
                sc = np.uint8(1) + (b % np.uint8(7))
            elif kind == 1:
                sc = np.uint8(8) + (b % np.uint8(0x77))
            else:
                sc = np.uint8(0x68) + (b & np.uint8(0xF))
            return np.where(c < 26, np.uint8(0), sc).astype(np.uint8)
        base = {0: 2.0 ** -1, 1: 2.0 ** -20, 2: 2.0 ** -14}[kind]
        w13, w13_sc = _bytes(g, (2 * Fd, H // 2)).copy(), scales((2 * Fd, H // 16))
        w2, w2_sc = _bytes(g, (H, Fd // 2)).copy(), scales((H, Fd // 16))
        gs = np.float32(base) * g.uniform(0.9, 1.1, size=3).astype(np.float32) * np.float32(gain)
        return dict(w13=w13, w13_sc=w13_sc, w2=w2, w2_sc=w2_sc, gs=gs.astype(np.float32))

    def elems(shape):
        b, c = _bytes(g, shape), _bytes(g, shape)
        sign = b & np.uint8(0x80)
        if kind == 0:
            mag = np.where(c < 26, np.uint8(0), np.uint8(1) + (b % np.uint8(7)))
        elif kind == 1:
            mag = np.where(c < 26, np.uint8(0),
                           np.where(c < 77, np.uint8(1) + (b % np.uint8(7)), np.uint8(8) + (b % np.uint8(0x77))))
        else:
            mag = np.where(c < 26, np.uint8(0), np.minimum(np.uint8(0x50) | (b & np.uint8(0x2F)), np.uint8(0x7E)))
        return (sign | mag).astype(np.uint8)

    def e8(shape):
        b = _bytes(g, shape)
        lo, n = {0: (121, 3), 1: (100, 27), 2: (112, 3)}[kind]
        return (np.uint8(lo) + (b % np.uint8(n))).astype(np.uint8)

    return dict(w13=elems((2 * Fd, H)), w13_sc=e8((2 * Fd, H // 32)), w2=elems((H, Fd)), w2_sc=e8((H, Fd // 32)))


def expert_direct_codes(seed: int, e: int, H: int, Fd: int, fmt: str, gain: float = 1.0,
                        edge: bool = False) -> dict:
    """Canonical-layout weights of expert e drawn directly as codes.
    gain multiplies the fp32 (NVFP4) scales or shifts the E8M0 scales by
    round(log2 gain) (MXFP8); it is used to push activations into the cap.
    edge: the edge-case draws described above (zero and subnormal scales and
    elements)."""
    if edge:
        if fmt not in ("nvfp4", "mxfp8"):
            raise ValueError(fmt)
        return _edge_codes(rng(seed, 5, e), e, H, Fd, fmt, gain)
    g = rng(seed, 4, e)
    if fmt == "nvfp4":
        w13 = _bytes(g, (2 * Fd, H // 2)).copy()
        w13_sc = _nv_scales(g, (2 * Fd, H // 16))
        w2 = _bytes(g, (H, Fd // 2)).copy()
        w2_sc = _nv_scales(g, (H, Fd // 16))
        gs = np.float32(2.0 ** -14) * g.uniform(0.9, 1.1, size=3).astype(np.float32) * np.float32(gain)
        return dict(w13=w13, w13_sc=w13_sc, w2=w2, w2_sc=w2_sc, gs=gs.astype(np.float32))
    if fmt == "mxfp8":
        sh = int(round(np.log2(gain)))
        return dict(w13=_mx_bytes(g, (2 * Fd, H)), w13_sc=_mx_scales(g, (2 * Fd, H // 32), sh),
                    w2=_mx_bytes(g, (H, Fd)), w2_sc=_mx_scales(g, (H, Fd // 32), sh))
    raise ValueError(fmt)

