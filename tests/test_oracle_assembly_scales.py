"""Pins of the oracle's expert-weight assembly and of the NVFP4 activation
scale readings (per row, per tensor, static).

Expert assembly: gate, up and down are drawn at magnitudes six orders apart,
so a swapped gate/up slice, a down matrix taken from the wrong array or a
wrong fp32-scale index breaks the round trip by orders of magnitude, far
outside each format's rounding bound (the bounds follow from the element
grids: an E2M1 value of a block is off by at most a sixth of the block
maximum times 1 + 2^-4 for the rounded block scale; an MXFP8 value by at most
an eighth of its block maximum, which the floor rule for the E8M0 scale
places in [256, 512) times the scale, so values above 448 saturate).

Activation scales: a row that holds the tensor maximum quantizes identically
under the row and tensor domains; a static scale that equals the row's own
scale reproduces the row domain; a static scale far too small saturates
every value to +-2688 * gs; and a dense evaluation of every expert
(torch float64, written here independently of the oracle's two-pass loop)
with the h scale taken over the selected pairs only equals the oracle's
per-tensor layer.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as L


def _blocks_max(v: np.ndarray, b: int) -> np.ndarray:
    R, K = v.shape
    return np.repeat(np.abs(v.reshape(R, K // b, b)).max(-1), b, axis=1)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_expert_assembly_round_trip_distinct_magnitudes(fmt):
    H, Fd = 256, 128
    g = np.random.default_rng(31)
    gate = (g.standard_normal((Fd, H)) * 1e-3).astype(np.float32)
    up = (g.standard_normal((Fd, H)) * 1.0).astype(np.float32)
    down = (g.standard_normal((H, Fd)) * 1e3).astype(np.float32)
    ew = L.quantize_expert_weights(fmt, gate, up, down)
    # canonical shapes: w13 = [gate rows; up rows], w2 = down
    nb = 16 if fmt == "nvfp4" else 32
    assert ew["w13"].shape == (2 * Fd, H // 2 if fmt == "nvfp4" else H)
    assert ew["w13_sc"].shape == (2 * Fd, H // nb)
    assert ew["w2"].shape == (H, Fd // 2 if fmt == "nvfp4" else Fd)
    assert ew["w2_sc"].shape == (H, Fd // nb)
    if fmt == "nvfp4":
        # one fp32 scale per matrix, in the order gate, up, down (reading R2)
        want = np.array([np.abs(m).max() for m in (gate, up, down)], dtype=np.float32) / np.float32(2688.0)
        assert np.array_equal(ew["gs"], want.astype(np.float32))
    G, U, D = L.dequantize_expert(fmt, ew)
    for orig, deq in ((gate, G), (up, U), (down, D)):
        o = orig.astype(np.float64)
        bound = _blocks_max(o, nb) * ((1 + 2.0 ** -4) / 6 if fmt == "nvfp4" else 1.0 / 8)
        assert np.all(np.abs(deq - o) <= bound * (1 + 1e-6))
        # and not trivially: every matrix keeps its own magnitude
        assert 0.5 < np.abs(deq).max() / np.abs(o).max() < 2.0


def test_expert_assembly_halves_are_independent():
    """Changing only the up matrix changes only rows F..2F-1 of w13 and gs[1]."""
    H, Fd = 128, 64
    g = np.random.default_rng(32)
    gate, up, down = (g.standard_normal(s).astype(np.float32) for s in ((Fd, H), (Fd, H), (H, Fd)))
    a = L.quantize_expert_weights("nvfp4", gate, up, down)
    b = L.quantize_expert_weights("nvfp4", gate, up * np.float32(3.0), down)
    assert np.array_equal(a["w13"][:Fd], b["w13"][:Fd]) and np.array_equal(a["w13_sc"][:Fd], b["w13_sc"][:Fd])
    assert not np.array_equal(a["gs"][1], b["gs"][1])
    assert a["gs"][0] == b["gs"][0] and a["gs"][2] == b["gs"][2]
    assert np.array_equal(a["w2"], b["w2"])


# ------------------------------------------------ NVFP4 activation scales --

def test_tensor_domain_equals_row_domain_on_the_max_row():
    g = np.random.default_rng(33)
    v = g.standard_normal((6, 128)).astype(np.float32)
    v[4] *= 50                                     # row 4 holds the tensor maximum
    cr, sr, gr = F.quantize_nvfp4(v, domain="row")
    ct, st, gt = F.quantize_nvfp4(v, domain="tensor")
    assert gt.ndim == 0 and gt == gr[4]
    assert np.array_equal(ct[4], cr[4]) and np.array_equal(st[4], sr[4])
    # the other rows are coarser under the shared scale: no larger block scale
    assert np.all(st[np.arange(6) != 4] <= sr[np.arange(6) != 4])


def test_static_scale_equal_to_the_row_scale_is_the_row_domain():
    g = np.random.default_rng(34)
    v = g.standard_normal((5, 64)).astype(np.float32) * np.float32(3.0)
    cr, sr, gr = F.quantize_nvfp4(v, domain="row")
    for r in range(5):
        c, s, gg = F.quantize_nvfp4(v[r:r + 1], domain="static", gs=gr[r])
        assert np.array_equal(c[0], cr[r]) and np.array_equal(s[0], sr[r]) and gg == gr[r]


def test_static_scale_saturates():
    v = np.array([[1e6, -1e6] + [0.0] * 14, [3.0] * 16], dtype=np.float32)
    c, s, gs = F.quantize_nvfp4(v, domain="static", gs=np.float32(1.0 / 64))
    d = F.dequantize_nvfp4(c, s, gs)
    # block scale clamps to 448, codes to +-6: +-2688 * gs
    assert d[0, 0] == 2688.0 / 64 and d[0, 1] == -2688.0 / 64 and np.all(d[0, 2:] == 0)
    assert np.all(d[1] == 3.0)                     # 3 = 6 * E4M3(3/(6/64)) * (1/64): in range, exact
    with pytest.raises(ValueError):
        F.quantize_nvfp4(v, domain="static", gs=np.float32(0.0))


def test_static_scale_lossless_on_its_grid():
    gsv = np.float32(2.0 ** -5)
    g = np.random.default_rng(35)
    codes = g.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, ::16] = 7                             # every block's maximum is 6: its scale is then sigma
    sig = F.E4M3_MAG[g.integers(40, 120, size=(4, 4))]
    v = (F.e2m1_decode(codes).reshape(4, 4, 16) * sig[..., None] * float(gsv)).reshape(4, 64).astype(np.float32)
    c, s, gs = F.quantize_nvfp4(v, domain="static", gs=gsv)
    assert np.array_equal(F.dequantize_nvfp4(c, s, gs), v.astype(np.float64))


def _small(seed, T, E, k, fmt="nvfp4", H=128, Fd=64, **kw):
    cfg = L.OracleConfig(hidden=H, ffn=Fd, num_experts=E, top_k=k, fmt=fmt, **kw)
    x = synth.tokens(seed, T, H)
    wr = synth.router_weight(seed, E, H, sigma=0.1)
    b = synth.router_bias(seed, E)
    ws = [L.quantize_expert_weights(fmt, *synth.expert_float_weights(seed, e, H, Fd, sigma=0.1)) for e in range(E)]
    return cfg, x, wr, b, ws


def test_single_pair_tensor_and_static_reduce_to_row():
    """One token and top-1: the x tensor is one row and the h tensor one
    (token, expert) row, so per-tensor equals per-row; a static pair equal to
    those two row scales (x first, h second) equals it too, and the swapped
    pair does not."""
    cfg, x, wr, b, ws = _small(36, 1, 4, 1)
    row = L.moe_layer(cfg, x, wr, b, ws)
    cfg_t = L.OracleConfig(**{**cfg.__dict__, "act_gs": "tensor"})
    assert np.array_equal(L.moe_layer(cfg_t, x, wr, b, ws)["out"], row["out"])
    e = int(row["topk_ids"][0, 0])
    xq = L.dequantize_rows("nvfp4", L.quantize_rows("nvfp4", F.bf16_bits_to_f32(x)))
    h = L.expert_gate_up(cfg, xq, L.dequantize_expert("nvfp4", ws[e]))
    x_gs = F.quantize_nvfp4(F.bf16_bits_to_f32(x))[2][0]
    h_gs = F.quantize_nvfp4(h)[2][0]
    assert x_gs != h_gs
    cfg_s = L.OracleConfig(**{**cfg.__dict__, "act_gs": "static", "act_gs_static": (x_gs, h_gs)})
    assert np.array_equal(L.moe_layer(cfg_s, x, wr, b, ws)["out"], row["out"])
    cfg_w = L.OracleConfig(**{**cfg.__dict__, "act_gs": "static", "act_gs_static": (h_gs, x_gs)})
    assert not np.array_equal(L.moe_layer(cfg_w, x, wr, b, ws)["out"], row["out"])


def _dense_per_tensor(cfg, x, wr, b, ws):
    """Every expert on every token in torch float64; x quantized with one
    scale over all tokens, h with one scale over the selected pairs."""
    r = L.route(cfg, x, wr, b)
    ids, tw = r["topk_ids"], r["topk_w"]
    xf = F.bf16_bits_to_f32(x)
    xq = torch.from_numpy(F.dequantize_nvfp4(*F.quantize_nvfp4(xf, domain="tensor")))
    T, E = x.shape[0], cfg.num_experts
    hs = []
    for e in range(E):
        gate, up, down = (torch.from_numpy(m) for m in L.dequantize_expert("nvfp4", ws[e]))
        gg, uu = (xq @ gate.T).float(), (xq @ up.T).float()
        hs.append(L.cap_swiglu(cfg, gg.numpy(), uu.numpy()))
    sel = np.zeros((E, T), dtype=bool)
    for j in range(cfg.top_k):
        sel[ids[:, j], np.arange(T)] = True
    amax = max(float(np.abs(hs[e][sel[e]]).max()) for e in range(E) if sel[e].any())
    h_gs = np.float32(np.float32(amax) / np.float32(2688.0))
    out = torch.zeros(T, cfg.hidden, dtype=torch.float64)
    for j in range(cfg.top_k):
        for t in range(T):
            e = int(ids[t, j])
            _, _, down = L.dequantize_expert("nvfp4", ws[e])
            hq = F.dequantize_nvfp4(*F.quantize_nvfp4(hs[e][t:t + 1], domain="static", gs=h_gs))
            y = (torch.from_numpy(hq) @ torch.from_numpy(down).T).float().double()[0]
            out[t] += float(tw[t, j]) * y
    return F.bf16_round_f64(out.numpy())


def test_per_tensor_layer_equals_dense_masked():
    cfg, x, wr, b, ws = _small(37, 12, 6, 2, act_gs="tensor")
    x = x.copy()
    x[3] = synth.to_bf16_bits(F.bf16_bits_to_f32(x[3]) * np.float32(40.0))   # one token sets the x scale
    got = L.moe_layer(cfg, x, wr, b, ws)
    assert np.array_equal(got["out"], _dense_per_tensor(cfg, x, wr, b, ws))
    row = L.moe_layer(L.OracleConfig(**{**cfg.__dict__, "act_gs": "row"}), x, wr, b, ws)
    assert not np.array_equal(got["out"], row["out"])
    with pytest.raises(ValueError):
        L.moe_layer(cfg, x, wr, b, ws, tokens=[0])


def test_mxfp8_ignores_act_gs():
    cfg, x, wr, b, ws = _small(38, 8, 6, 2, fmt="mxfp8")
    a = L.moe_layer(cfg, x, wr, b, ws)["out"]
    for mode in ("tensor", "static"):
        c = L.OracleConfig(**{**cfg.__dict__, "act_gs": mode, "act_gs_static": (0.5, 0.25)})
        assert np.array_equal(L.moe_layer(c, x, wr, b, ws)["out"], a)
