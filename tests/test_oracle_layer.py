"""Pins of the oracle's router, dispatch, expert FFN and combine.

The references here are computed differently from the oracle: full sorts in
pure Python, torch float64 library ops (matmul, sigmoid, silu, tanh, clamp),
a dense evaluation of every expert masked to the top-k, and invariances the
definition implies (expert permutation, token independence, expert-parallel
partial sums).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as L


def _small(seed=0, T=24, H=128, E=12, k=3, Fd=64, fmt="mxfp8", **kw):
    cfg = L.OracleConfig(hidden=H, ffn=Fd, num_experts=E, top_k=k, fmt=fmt, **kw)
    x = synth.tokens(seed, T, H)
    wr = synth.router_weight(seed, E, H, sigma=0.1)
    b = synth.router_bias(seed, E)
    ws = [L.quantize_expert_weights(fmt, *synth.expert_float_weights(seed, e, H, Fd, sigma=0.1))
          for e in range(E)]
    return cfg, x, wr, b, ws


# ----------------------------------------------------------------- router --

def test_router_logits_and_scores_match_torch_f64():
    cfg, x, wr, b, _ = _small()
    r = L.route(cfg, x, wr, b)
    xt = torch.from_numpy(F.bf16_bits_to_f32(x).astype(np.float64))
    wt = torch.from_numpy(F.bf16_bits_to_f32(wr).astype(np.float64))
    z = (xt @ wt.T).to(torch.float32)
    assert torch.equal(torch.from_numpy(r["logits"]), z)
    s = torch.sigmoid(z.to(torch.float64)).to(torch.float32)
    assert torch.equal(torch.from_numpy(r["scores"]), s)


def test_topk_matches_python_sort():
    cfg, x, wr, b, _ = _small(seed=3, T=40, E=32, k=5)
    r = L.route(cfg, x, wr, b)
    sel = r["sel"]
    for t in range(sel.shape[0]):
        order = sorted(range(sel.shape[1]), key=lambda e: (-float(sel[t, e]), e))
        assert list(r["topk_ids"][t]) == order[:5]
        gap = float(sel[t, order[4]]) - float(sel[t, order[5]])
        assert r["near_tie"][t] == (gap < 1e-6)


def test_exact_tie_goes_to_lower_index():
    cfg, x, wr, b, _ = _small(seed=4, E=8, k=2)
    wr = wr.copy()
    b = b.copy()
    wr[5] = wr[2]
    b[5] = b[2] = 10.0              # experts 2 and 5 always on top, exactly tied
    r = L.route(cfg, x, wr, b)
    assert np.all(r["topk_ids"][:, 0] == 2) and np.all(r["topk_ids"][:, 1] == 5)
    cfg1 = L.OracleConfig(hidden=cfg.hidden, ffn=cfg.ffn, num_experts=8, top_k=1, fmt="mxfp8")
    r1 = L.route(cfg1, x, wr, b)
    assert np.all(r1["topk_ids"][:, 0] == 2) and np.all(r1["near_tie"])


def test_bias_only_selects():
    cfg, x, wr, b, _ = _small(seed=5, E=16, k=4)
    r = L.route(cfg, x, wr, b)
    r0 = L.route(cfg, x, wr, np.zeros_like(b))
    s = torch.sigmoid(torch.from_numpy(r0["logits"]).double()).float().numpy()
    w = np.take_along_axis(s, r["topk_ids"].astype(np.int64), 1).astype(np.float64)
    assert np.allclose(r["topk_w"], w / w.sum(1, keepdims=True), rtol=1e-6, atol=0)
    assert np.allclose(r["topk_w"].sum(1), 1.0, atol=1e-6)


def test_routed_scale_and_no_norm():
    cfg, x, wr, b, _ = _small(seed=6, E=16, k=4, norm_topk=False, routed_scale=2.5)
    r = L.route(cfg, x, wr, b)
    w = np.take_along_axis(r["scores"], r["topk_ids"].astype(np.int64), 1)
    assert np.allclose(r["topk_w"], 2.5 * w.astype(np.float64), rtol=1e-7)


# --------------------------------------------------------------- dispatch --

@pytest.mark.parametrize("begin,nloc", [(0, None), (4, 5)])
def test_dispatch_matches_python_sort(begin, nloc):
    g = np.random.default_rng(7)
    T, k, E = 50, 4, 16
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    cfg = L.OracleConfig(hidden=32, ffn=32, num_experts=E, top_k=k, fmt="mxfp8", expert_begin=begin, num_local=nloc)
    off, sp, pos = L.dispatch(cfg, ids)
    lo, hi = begin, begin + (E if nloc is None else nloc)
    ref = sorted([(int(ids.ravel()[p]), p) for p in range(T * k) if lo <= ids.ravel()[p] < hi])
    assert list(sp) == [p for _, p in ref]
    assert off[0] == 0 and off[-1] == len(ref)
    for e in range(lo, hi):
        seg = sp[off[e - lo]:off[e - lo + 1]]
        assert np.all(ids.ravel()[seg] == e)
    assert np.all(pos[sp] == np.arange(len(sp)))
    assert np.all((pos == -1) == ~((ids.ravel() >= lo) & (ids.ravel() < hi)))


# ---------------------------------------------------------- cap / SwiGLU --

def test_cap_swiglu_forms_match_torch():
    g = np.random.default_rng(8)
    a = (g.standard_normal(5000) * 6).astype(np.float32)
    u = (g.standard_normal(5000) * 6).astype(np.float32)
    at, ut = torch.from_numpy(a).double(), torch.from_numpy(u).double()
    c = 7.0
    cfg = L.OracleConfig(hidden=32, ffn=32, num_experts=2, top_k=1, fmt="mxfp8", cap=c)
    silu = torch.nn.functional.silu
    for form, ref in [
        (L.CAP_NONE, silu(at) * ut),
        (L.CAP_SOFT_GATE_UP, silu(c * torch.tanh(at / c)) * (c * torch.tanh(ut / c))),
        (L.CAP_HARD_GATE_UP, silu(torch.clamp(at, max=c)) * torch.clamp(ut, -c, c)),
        (L.CAP_SOFT_OUT, c * torch.tanh(silu(at) * ut / c)),
    ]:
        cfg.cap_form = form
        got = torch.from_numpy(L.cap_swiglu(cfg, a, u)).double()
        assert torch.allclose(got, ref.float().double(), rtol=2e-7, atol=1e-30), form


def test_large_cap_is_plain_swiglu():
    g = np.random.default_rng(9)
    a = (g.standard_normal(1000)).astype(np.float32)
    u = (g.standard_normal(1000)).astype(np.float32)
    cfg = L.OracleConfig(hidden=32, ffn=32, num_experts=2, top_k=1, fmt="mxfp8", cap=1e12)
    ref = (torch.nn.functional.silu(torch.from_numpy(a).double()) * torch.from_numpy(u).double()).float().numpy()
    assert np.array_equal(L.cap_swiglu(cfg, a, u), ref)


# ------------------------------------------------------------ whole layer --

def _dense_masked(cfg, x, wr, b, ws):
    """Every expert on every token (torch float64), masked to the top-k."""
    r = L.route(cfg, x, wr, b)
    ids, tw = r["topk_ids"], r["topk_w"]
    if cfg.fmt == "mxfp8":
        xq = torch.from_numpy(F.dequantize_mxfp8(*F.quantize_mxfp8(F.bf16_bits_to_f32(x))))
    else:
        xq = torch.from_numpy(F.dequantize_nvfp4(*F.quantize_nvfp4(F.bf16_bits_to_f32(x))))
    T = x.shape[0]
    E = cfg.num_experts
    Y = torch.zeros(E, T, cfg.hidden, dtype=torch.float64)
    for e in range(E):
        gate, up, down = (torch.from_numpy(m) for m in L.dequantize_expert(cfg.fmt, ws[e]))
        gg = (xq @ gate.T).float()
        uu = (xq @ up.T).float()
        h = torch.from_numpy(L.cap_swiglu(cfg, gg.numpy(), uu.numpy()))
        if cfg.fmt == "mxfp8":
            hq = torch.from_numpy(F.dequantize_mxfp8(*F.quantize_mxfp8(h.numpy())))
        else:
            hq = torch.from_numpy(F.dequantize_nvfp4(*F.quantize_nvfp4(h.numpy())))
        Y[e] = (hq @ down.T).float().double()
    out = torch.zeros(T, cfg.hidden, dtype=torch.float64)
    loc = cfg.local
    for j in range(cfg.top_k):
        m = torch.tensor([(int(i) in loc) for i in ids[:, j]], dtype=torch.float64)[:, None]
        out = out + m * torch.from_numpy(tw[:, j].astype(np.float64))[:, None] * Y[torch.from_numpy(ids[:, j].astype(np.int64)), torch.arange(T)]
    return F.bf16_round_f64(out.numpy())


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_sparse_equals_dense_masked(fmt):
    cfg, x, wr, b, ws = _small(seed=11, fmt=fmt)
    got = L.moe_layer(cfg, x, wr, b, ws)["out"]
    assert np.array_equal(got, _dense_masked(cfg, x, wr, b, ws))


def test_expert_parallel_share_masks_other_experts():
    cfg, x, wr, b, ws = _small(seed=12, E=12, k=3)
    cfg.expert_begin, cfg.num_local = 4, 5
    got = L.moe_layer(cfg, x, wr, b, ws[4:9])
    assert np.array_equal(got["out"], _dense_masked(cfg, x, wr, b, ws))


def test_expert_parallel_shares_sum_to_full():
    cfg, x, wr, b, ws = _small(seed=13, E=12, k=3)
    full = L.moe_layer(cfg, x, wr, b, ws)
    acc = np.zeros((x.shape[0], cfg.hidden))
    for lo in range(0, 12, 4):
        c = L.OracleConfig(**{**cfg.__dict__, "expert_begin": lo, "num_local": 4})
        part = L.moe_layer(c, x, wr, b, ws[lo:lo + 4])
        acc += (part["y"].astype(np.float64) * part["topk_w"][..., None] * part["have"][..., None]).sum(1)
    ref = (full["y"].astype(np.float64) * full["topk_w"][..., None]).sum(1)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-300)


def test_expert_permutation_invariance():
    cfg, x, wr, b, ws = _small(seed=14, E=10, k=3)
    perm = np.random.default_rng(0).permutation(10)           # new expert i = old perm[i]
    out0 = L.moe_layer(cfg, x, wr, b, ws)
    out1 = L.moe_layer(cfg, x, wr[perm], b[perm], [ws[p] for p in perm])
    inv = np.argsort(perm)
    assert np.array_equal(out1["topk_ids"], inv[out0["topk_ids"]])
    assert np.array_equal(out1["out"], out0["out"])


def test_token_independence():
    cfg, x, wr, b, ws = _small(seed=15, T=12, fmt="nvfp4")
    x2 = x.copy()
    x2[1:] = synth.tokens(99, 11, cfg.hidden)
    a = L.moe_layer(cfg, x, wr, b, ws)["out"][0]
    c = L.moe_layer(cfg, x2, wr, b, ws)["out"][0]
    assert np.array_equal(a, c)
    sub = L.moe_layer(cfg, x, wr, b, ws, tokens=[3, 7])["out"]
    assert np.array_equal(sub, L.moe_layer(cfg, x, wr, b, ws)["out"][[3, 7]])


def test_all_experts_is_dense_sigmoid_mixture():
    # top_k = E with normalisation: every expert contributes s_e / sum(s)
    cfg, x, wr, b, ws = _small(seed=16, E=6, k=6)
    res = L.moe_layer(cfg, x, wr, b, ws)
    s = torch.sigmoid(torch.from_numpy(res["route"]["logits"]).double()).float().double()
    wts = s / s.sum(1, keepdim=True)
    dense = _dense_masked(cfg, x, wr, b, ws)
    assert np.array_equal(res["out"], dense)
    ids = res["topk_ids"].astype(np.int64)
    assert np.allclose(res["topk_w"], np.take_along_axis(wts.numpy(), ids, 1), rtol=1e-6)


def test_routing_replay_overrides_router():
    cfg, x, wr, b, ws = _small(seed=17, E=8, k=2)
    T = x.shape[0]
    ids = np.tile(np.array([[6, 1]], dtype=np.int32), (T, 1))
    tw = np.full((T, 2), 0.5, dtype=np.float32)
    res = L.moe_layer(cfg, x, wr, b, ws, topk_ids=ids, topk_w=tw)
    xq = F.dequantize_mxfp8(*F.quantize_mxfp8(F.bf16_bits_to_f32(x)))
    y6, _ = L.expert_forward(cfg, xq, L.dequantize_expert("mxfp8", ws[6]))
    y1, _ = L.expert_forward(cfg, xq, L.dequantize_expert("mxfp8", ws[1]))
    ref = F.bf16_round_f64(0.5 * y6.astype(np.float64) + 0.5 * y1.astype(np.float64))
    assert np.array_equal(res["out"], ref)


def test_expert_matches_plain_f64_ffn_on_representable_inputs():
    """With x and weights exactly on their grids and the cap off, gate/up equal a
    plain float64 FFN; the down projection sees h after its own quantization."""
    H, Fd = 64, 32
    cfg = L.OracleConfig(hidden=H, ffn=Fd, num_experts=1, top_k=1, fmt="mxfp8", cap_form=L.CAP_NONE)
    g = np.random.default_rng(18)
    gate, up, down = (m * 0.1 for m in synth.expert_float_weights(1, 0, H, Fd))
    ew = L.quantize_expert_weights("mxfp8", gate, up, down)
    G, U, D = L.dequantize_expert("mxfp8", ew)
    x = g.integers(-4, 5, size=(5, H)).astype(np.float64)          # exact in E4M3 with any block scale
    x[:, 0] = 256                                                   # block max 256 -> scale 2^0
    x[:, 32] = 256
    xb = synth.to_bf16_bits(x.astype(np.float32))
    xq = F.dequantize_mxfp8(*F.quantize_mxfp8(F.bf16_bits_to_f32(xb)))
    assert np.array_equal(xq, x)
    y, h = L.expert_forward(cfg, xq, (G, U, D))
    gg = torch.from_numpy(x) @ torch.from_numpy(G).T
    uu = torch.from_numpy(x) @ torch.from_numpy(U).T
    href = (torch.nn.functional.silu(gg.float().double()) * uu.float().double()).float().numpy()
    assert np.array_equal(h, href)
    hq = F.dequantize_mxfp8(*F.quantize_mxfp8(h))
    assert np.array_equal(y, (torch.from_numpy(hq) @ torch.from_numpy(D).T).float().numpy())


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_worker_pool_matches_one_process(fmt):
    """Experts evaluated by forked worker processes give the serial result bit
    for bit (the per-expert arithmetic is unchanged; the combine is a
    fixed-order sum)."""
    cfg, x, wr, b, ws = _small(seed=16, E=12, k=3, fmt=fmt)
    one = L.moe_layer(cfg, x, wr, b, ws)
    pool = L.moe_layer(cfg, x, wr, b, ws, workers=3)
    for key in ("out", "y", "topk_ids", "topk_w"):
        assert np.array_equal(np.asarray(one[key]).view(np.uint8), np.asarray(pool[key]).view(np.uint8)), key


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_topk_slot_permutation_invariance(fmt):
    """Permuting each token's k slots (ids and gate weights together) leaves
    the layer output unchanged: the combine is a sum over the chosen experts
    (accumulated in float64, rounded once to bf16)."""
    cfg, x, wr, b, ws = _small(seed=17, E=12, k=4, fmt=fmt)
    r = L.moe_layer(cfg, x, wr, b, ws)
    g = np.random.default_rng(5)
    perm = np.stack([g.permutation(cfg.top_k) for _ in range(x.shape[0])])
    ids = np.take_along_axis(r["topk_ids"], perm, axis=1)
    tw = np.take_along_axis(r["topk_w"], perm, axis=1)
    p = L.moe_layer(cfg, x, wr, b, ws, topk_ids=ids, topk_w=tw)
    assert not np.array_equal(ids, r["topk_ids"])
    assert np.array_equal(p["out"], r["out"])
