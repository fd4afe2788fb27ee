"""moe_encode_weights / moe_decode_weights on the GPU vs the oracle's encoder.

Codes, block scales and per-matrix fp32 scales must be bit-identical to the
oracle's canonical encoding of the same fp32 (or bf16) weights; decoded fp32
values must equal the oracle's exact float64 values rounded once to fp32.
Cases: Gaussian experts at small and Inkling sizes, bf16 input, a zero
matrix, one huge and one tiny matrix (saturating / subnormal block scales),
and ragged block contents.
"""
import zlib

import numpy as np
import pytest

from oracle import layer as L

pytestmark = pytest.mark.gpu


def experts(rng, n, H, Fd, kind="gauss"):
    out = []
    for e in range(n):
        g = rng.normal(0, 0.02, (Fd, H)).astype(np.float32)
        u = rng.normal(0, 0.02, (Fd, H)).astype(np.float32)
        d = rng.normal(0, 0.02, (H, Fd)).astype(np.float32)
        if kind == "edge":
            if e == 0:
                g[:] = 0.0                                  # zero matrix: gs = 1, all codes 0
            if e == 1:
                u *= np.float32(3e36)                        # huge values
                d *= np.float32(1e-33)                       # tiny values (subnormal block scales)
            g[:, ::7] = 0.0                                  # ragged zeros inside blocks
            u[::5, :16] = np.float32(448.0 * 6.0) * np.sign(u[::5, :16])
        out.append((g, u, d))
    return out


def encode_gpu(bse, fmt, ex, dtype="f32"):
    import torch
    n = len(ex)
    Fd, H = ex[0][0].shape
    gu = np.stack([np.stack([g, u]) for g, u, _ in ex])      # [n, 2, F, H]
    dn = np.stack([d for _, _, d in ex])                      # [n, H, F]
    t = lambda a: torch.from_numpy(a).cuda()                 # noqa: E731
    wg, wd = t(gu.reshape(2 * n, Fd, H)), t(dn)
    if dtype == "bf16":
        wg, wd = wg.to(torch.bfloat16), wd.to(torch.bfloat16)
    nv = fmt == "nvfp4"
    c13 = torch.empty((2 * n, Fd, H // 2 if nv else H), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((2 * n, Fd, H // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    c2 = torch.empty((n, H, Fd // 2 if nv else Fd), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((n, H, Fd // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    gs = torch.full((n, 3), -1.0, dtype=torch.float32, device="cuda") if nv else None
    ws = torch.empty(2 * n, dtype=torch.int32, device="cuda") if nv else None
    bse.encode_weights(fmt, wg, c13, s13, gs=gs, gs_group=2, gs_stride=3, ws=ws)
    # the down scales sit at gs[e][2]: a flat view from element 2, stride 3
    bse.encode_weights(fmt, wd, c2, s2, gs=gs.view(-1)[2:] if nv else None, gs_group=1, gs_stride=3, ws=ws)
    torch.cuda.synchronize()
    res = dict(w13=c13.cpu().numpy().reshape(n, 2 * Fd, -1), w13_sc=s13.cpu().numpy().reshape(n, 2 * Fd, -1),
               w2=c2.cpu().numpy(), w2_sc=s2.cpu().numpy())
    if nv:
        res["gs"] = gs.cpu().numpy()
    return res, (c13, s13, c2, s2, gs)


def as_oracle_input(ex, dtype):
    if dtype == "f32":
        return ex
    import torch
    r = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()   # noqa: E731
    return [(r(g), r(u), r(d)) for g, u, d in ex]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
@pytest.mark.parametrize("kind,dtype,H,Fd,n", [
    ("gauss", "f32", 256, 128, 3), ("gauss", "bf16", 512, 256, 2), ("edge", "f32", 256, 128, 3),
    ("gauss", "bf16", 4608, 2304, 1),
])
def test_encode_matches_oracle_bit_exact(gpu_lib, fmt, kind, dtype, H, Fd, n):
    rng = np.random.default_rng(zlib.crc32(repr((fmt, kind, dtype, H)).encode()))
    ex = experts(rng, n, H, Fd, kind)
    got, _ = encode_gpu(gpu_lib, fmt, ex, dtype)
    for e, (g, u, d) in enumerate(as_oracle_input(ex, dtype)):
        ref = L.quantize_expert_weights(fmt, g, u, d)
        for key in ("w13", "w13_sc", "w2", "w2_sc"):
            assert np.array_equal(got[key][e], np.asarray(ref[key])), (e, key)
        if fmt == "nvfp4":
            assert np.array_equal(got["gs"][e].view(np.uint32), np.asarray(ref["gs"], np.float32).view(np.uint32)), e


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_decode_matches_oracle(gpu_lib, fmt):
    import torch
    rng = np.random.default_rng(7)
    n, H, Fd = 2, 256, 128
    ex = experts(rng, n, H, Fd, "edge")
    _, (c13, s13, c2, s2, gs) = encode_gpu(gpu_lib, fmt, ex)
    o13 = torch.empty((2 * n, Fd, H), dtype=torch.float32, device="cuda")
    o2 = torch.empty((n, H, Fd), dtype=torch.float32, device="cuda")
    gpu_lib.decode_weights(fmt, c13, s13, o13, gs=gs, gs_group=2, gs_stride=3)
    gpu_lib.decode_weights(fmt, c2, s2, o2, gs=gs.view(-1)[2:] if gs is not None else None, gs_group=1,
                           gs_stride=3)
    torch.cuda.synchronize()
    o13, o2 = o13.cpu().numpy(), o2.cpu().numpy()
    for e, (g, u, d) in enumerate(ex):
        gq, uq, dq = L.dequantize_expert(fmt, L.quantize_expert_weights(fmt, g, u, d))
        with np.errstate(over="ignore"):
            assert np.array_equal(o13[2 * e], gq.astype(np.float32))
            assert np.array_equal(o13[2 * e + 1], uq.astype(np.float32))
            assert np.array_equal(o2[e], dq.astype(np.float32))
