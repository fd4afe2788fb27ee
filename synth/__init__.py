"""Seeded synthetic inputs for the routed-expert MoE layer.

Shared by the tests, the benchmark and the smoke check.  This module only
draws random numbers and lays them out; it holds none of the layer's
arithmetic (no quantization, routing or matmul).  Every array is a pure
function of (seed, stream, ...) through numpy's PCG64 with a SeedSequence, so
any single expert can be regenerated on its own.

Streams: 0 = tokens x, 1 = router weight, 2 = router bias, (3, e) = float
weights of expert e, (4, e) = direct-code weights of expert e.
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


# Direct-code weights: random valid encodings drawn straight from fixed
# distributions (no quantizer involved), sized so that an element's RMS is
# about 0.02 like the float recipe.  Used where encoding hundreds of
# full-size experts from floats would take minutes.
#   NVFP4: every nibble uniform over the 16 E2M1 codes; block-scale bytes
#          uniform over E4M3 codes 0x68..0x7E (64 .. 448); fp32 scale per
#          matrix 2^-15 * U(0.9, 1.1).
#   MXFP8: E4M3 bytes with a random sign, exponent field uniform in 10..15 and
#          a uniform mantissa (0x7F/0xFF remapped to 0x7E/0xFE); E8M0 scale
#          bytes uniform in 112..114 (2^-15 .. 2^-13).
NV_SCALE_LO, NV_SCALE_HI = 0x68, 0x7E
MX_EXP_LO, MX_EXP_HI = 10, 15
MX_SCALE_LO, MX_SCALE_HI = 112, 114


def _mx_bytes(g: np.random.Generator, shape) -> np.ndarray:
    sign = g.integers(0, 2, size=shape, dtype=np.uint8) << 7
    ex = g.integers(MX_EXP_LO, MX_EXP_HI + 1, size=shape, dtype=np.uint8) << 3
    man = g.integers(0, 8, size=shape, dtype=np.uint8)
    b = sign | ex | man
    b[(b & 0x7F) == 0x7F] -= 1
    return b


def expert_direct_codes(seed: int, e: int, H: int, Fd: int, fmt: str, gain: float = 1.0) -> dict:
    """Canonical-layout weights of expert e drawn directly as codes.
    gain multiplies the fp32 (NVFP4) scales or shifts the E8M0 scales by
    round(log2 gain) (MXFP8); it is used to push activations into the cap."""
    g = rng(seed, 4, e)
    if fmt == "nvfp4":
        w13 = g.integers(0, 256, size=(2 * Fd, H // 2), dtype=np.uint8)
        w13_sc = g.integers(NV_SCALE_LO, NV_SCALE_HI + 1, size=(2 * Fd, H // 16), dtype=np.uint8)
        w2 = g.integers(0, 256, size=(H, Fd // 2), dtype=np.uint8)
        w2_sc = g.integers(NV_SCALE_LO, NV_SCALE_HI + 1, size=(H, Fd // 16), dtype=np.uint8)
        gs = (np.float32(2.0 ** -15) * g.uniform(0.9, 1.1, size=3).astype(np.float32) * np.float32(gain))
        return dict(w13=w13, w13_sc=w13_sc, w2=w2, w2_sc=w2_sc, gs=gs.astype(np.float32))
    if fmt == "mxfp8":
        sh = int(round(np.log2(gain)))
        w13 = _mx_bytes(g, (2 * Fd, H))
        w13_sc = (g.integers(MX_SCALE_LO, MX_SCALE_HI + 1, size=(2 * Fd, H // 32)) + sh).astype(np.uint8)
        w2 = _mx_bytes(g, (H, Fd))
        w2_sc = (g.integers(MX_SCALE_LO, MX_SCALE_HI + 1, size=(H, Fd // 32)) + sh).astype(np.uint8)
        return dict(w13=w13, w13_sc=w13_sc, w2=w2, w2_sc=w2_sc)
    raise ValueError(fmt)

