"""moe_quantize_act on the GPU vs the oracle: codes, block scales and row
scales must be bit-identical (integer/byte output)."""
import numpy as np
import pytest

import synth
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _edge_rows_bf16(H, seed=0):
    g = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(H, np.float32))                                  # zero row
    r = g.standard_normal(H).astype(np.float32); r[: H // 2] = 0; rows.append(r)   # zero blocks
    rows.append((np.sign(g.standard_normal(H)) * g.uniform(1e37, 3.3e38, H)).astype(np.float32))  # huge, finite
    rows.append(g.standard_normal(H).astype(np.float32) * np.float32(1e-38))       # tiny / subnormal
    rows.append(np.full(H, 9.2e-41, np.float32))                          # all bf16 subnormal
    # exact E2M1 / E4M3 midpoints at unit scales
    mid = np.resize(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -5.0], np.float32), H)
    rows.append(mid)
    rows.append(-np.abs(g.standard_normal(H).astype(np.float32)) * np.float32(1e-3))  # rounds to -0 often
    r = g.standard_normal(H).astype(np.float32); r[::7] = -0.0; rows.append(r)
    rows.append(np.exp(g.uniform(-80, 80, H)).astype(np.float32) * np.sign(g.standard_normal(H)).astype(np.float32))
    return synth.to_bf16_bits(np.stack(rows))


def _f32_rows(H, seed=1):
    g = np.random.default_rng(seed)
    a = (g.standard_normal((37, H)) * np.exp(g.uniform(-30, 30, (37, 1)))).astype(np.float32)
    a[0] = 0
    a[1, :64] = -0.0
    a[2] = np.float32(1e-42)
    a[3] *= np.float32(1e5)
    return a


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
@pytest.mark.parametrize("H", [256, 4608])
def test_quantize_bf16_rows_bit_exact(gpu_lib, fmt, H):
    import torch
    x = np.concatenate([synth.tokens(3, 61, H), _edge_rows_bf16(H)])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    R = x.shape[0]
    nv = fmt == "nvfp4"
    codes = torch.empty((R, H // 2 if nv else H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, H // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    gs = torch.empty(R, dtype=torch.float32, device="cuda") if nv else None
    gpu_lib.quantize_act(fmt, xt, codes, scales, gs)
    torch.cuda.synchronize()
    xf = F.bf16_bits_to_f32(x)
    if nv:
        c, s, g = F.quantize_nvfp4(xf, domain="row")
        assert np.array_equal(gs.cpu().numpy().view(np.uint32), g.view(np.uint32))
    else:
        c, s = F.quantize_mxfp8(xf)
    assert np.array_equal(scales.cpu().numpy(), s)
    assert np.array_equal(codes.cpu().numpy(), c)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_quantize_f32_rows_bit_exact(gpu_lib, fmt):
    import torch
    H = 2304
    x = _f32_rows(H)
    R = x.shape[0]
    nv = fmt == "nvfp4"
    codes = torch.empty((R, H // 2 if nv else H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, H // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    gs = torch.empty(R, dtype=torch.float32, device="cuda") if nv else None
    gpu_lib.quantize_act(fmt, torch.from_numpy(x).cuda(), codes, scales, gs)
    torch.cuda.synchronize()
    if nv:
        c, s, g = F.quantize_nvfp4(x, domain="row")
        assert np.array_equal(gs.cpu().numpy().view(np.uint32), g.view(np.uint32))
    else:
        c, s = F.quantize_mxfp8(x)
    assert np.array_equal(scales.cpu().numpy(), s)
    assert np.array_equal(codes.cpu().numpy(), c)


def test_quantize_prefill_rows_bit_exact(gpu_lib):
    """16384 Inkling-width rows (the prefill chunk) in NVFP4, checked in full."""
    import torch
    w = synth.WORKLOADS["prefill_nvfp4"]
    x = synth.tokens(w.seed, w.tokens, w.hidden)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    R, H = x.shape
    codes = torch.empty((R, H // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, H // 16), dtype=torch.uint8, device="cuda")
    gs = torch.empty(R, dtype=torch.float32, device="cuda")
    gpu_lib.quantize_act("nvfp4", xt, codes, scales, gs)
    torch.cuda.synchronize()
    for lo in range(0, R, 4096):
        c, s, g = F.quantize_nvfp4(F.bf16_bits_to_f32(x[lo:lo + 4096]), domain="row")
        assert np.array_equal(gs[lo:lo + 4096].cpu().numpy(), g)
        assert np.array_equal(scales[lo:lo + 4096].cpu().numpy(), s)
        assert np.array_equal(codes[lo:lo + 4096].cpu().numpy(), c)


def _shared_scale_case(gpu_lib, mode, x, dtype, site, H):
    """GPU quantize_act with one scale for all rows vs the oracle's tensor /
    static domains; returns nothing, asserts bit-identity."""
    import torch
    R = x.shape[0]
    static = (np.float32(1.37 / 8), np.float32(0.0123))
    cfg = gpu_lib.Config(fmt="nvfp4", act_gs=gpu_lib.ACT_GS_PER_TENSOR if mode == "tensor" else gpu_lib.ACT_GS_STATIC,
                         act_gs_static=(float(static[0]), float(static[1])))
    xt = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(x)).cuda()
    codes = torch.empty((R, H // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, H // 16), dtype=torch.uint8, device="cuda")
    gs = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.ACT_GS_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    gpu_lib.quantize_act(cfg, xt, codes, scales, gs, site=site, ws=ws if mode == "tensor" else None)
    torch.cuda.synchronize()
    xf = F.bf16_bits_to_f32(x) if dtype == "bf16" else x
    if mode == "tensor":
        c, s, g = F.quantize_nvfp4(xf, domain="tensor")
    else:
        c, s, g = F.quantize_nvfp4(xf, domain="static", gs=static[site])
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), np.full(R, g, np.float32).view(np.uint32))
    assert np.array_equal(scales.cpu().numpy(), s)
    assert np.array_equal(codes.cpu().numpy(), c)


@pytest.mark.parametrize("site", [0, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["tensor", "static"])
def test_quantize_nvfp4_shared_scale_bit_exact(gpu_lib, mode, dtype, site):
    """Per-tensor and static NVFP4 activation scales (the alternatives of the
    per-row reading): codes, block scales and the shared fp32 scale
    bit-identical to the oracle, including saturating rows."""
    if dtype == "bf16":
        H = 4608
        x = np.concatenate([synth.tokens(5, 40, H), _edge_rows_bf16(H)])
    else:
        H = 2304
        x = _f32_rows(H)
    _shared_scale_case(gpu_lib, mode, x, dtype, site, H)


def test_quantize_nvfp4_per_tensor_many_rows(gpu_lib):
    """A tensor of 5000 Inkling-width rows: the two-pass maximum runs over 256
    partial slices; one row holds the tensor maximum."""
    x = synth.tokens(9, 5000, 4608)
    x[3117, 100] = synth.to_bf16_bits(np.array([[-40.0]], np.float32))[0, 0]
    _shared_scale_case(gpu_lib, "tensor", x, "bf16", 0, 4608)
