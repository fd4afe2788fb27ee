"""GPU parity beyond the basic shapes: every router kernel variant, the
Inkling-size workloads compared on every token, the large-M kernels on every
row position of the prefill chunk, and edge-case activations and weights.

Tolerance as everywhere: max|gpu - oracle| / max|oracle| <= 2e-2 on the bf16
layer output (routing replayed into the oracle); routing sets bit-exact away
from near ties.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L

from _util import (ORACLE_WORKERS, OUT_RTOL, ExpertSource, bf16_to_f64, inputs, lib_cfg, oracle_cfg, rel_err,
                   stack_local, to_dev)
from test_gpu_route_dispatch import _check_route, _run_route

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ router --
# Router kernel variants by batch: split-K GEMV tiles of 16 / 32 / 64 tokens
# with 6 / 4 / 2 K slices up to 256 tokens, then 128 x 128 LDS tiles with as
# many K slices as keep the grid within 256 workgroups, at least 2 (6 at 300
# tokens; 5 at 2048 -- slices of 14 and 15 steps, the odd last step skipped;
# 2 at 4096 and 16384); top-k with 1 / 2 / 4 / 8 / 16 experts per lane.
ROUTER_CASES = [
    (24, 384, 8), (100, 384, 8), (200, 384, 8), (300, 384, 8), (2048, 384, 8), (4096, 384, 8),
    (50, 40, 4), (130, 100, 6), (37, 200, 8), (300, 600, 8), (70, 1000, 8), (5, 64, 3),
]


@pytest.mark.parametrize("T,E,k", ROUTER_CASES)
def test_route_every_kernel_variant(gpu_lib, T, E, k):
    w = synth.Workload("r", "router", T, 4608, E, k, 2304, "nvfp4", 50 + T % 7 + E % 5)
    got = _run_route(gpu_lib, w, T)
    ties = _check_route(w, *got)
    assert ties <= max(2, T // 20)


# ------------------------------------------------- Inkling size, all tokens --

def _run(bse, w, ids=None, tw=None, edge=False, gain=1.0):
    """Route (unless ids/tw are given) and run the forward on the GPU for
    workload w with its local experts; returns host arrays."""
    import torch
    x, wr, b = inputs(w)
    T = x.shape[0]
    cfg = lib_cfg(bse, w, max_tokens=T)
    n = w.experts if w.num_local is None else w.num_local
    src = ExpertSource(w, gain, edge)
    ews = [src(w.expert_begin + i) for i in range(n)]
    keys = ("w13", "w13_sc", "w2", "w2_sc") + (("gs",) if w.fmt == "nvfp4" else ())
    wd = {kk: to_dev(np.stack([np.asarray(e[kk]) for e in ews])) for kk in keys}
    del ews
    wd = bse.prepare_weights(cfg, wd)
    ws = bse.workspace(cfg)
    xt = to_dev(x.view(np.int16), torch.bfloat16)
    if ids is None:
        idt = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        twt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
        bse.route(cfg, xt, to_dev(wr.view(np.int16), torch.bfloat16), to_dev(b), idt, twt, None, ws)
    else:
        idt, twt = to_dev(ids), to_dev(tw)
    out = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
    bse.forward(cfg, xt, idt, twt, wd, out, ws)
    again = torch.empty_like(out)
    bse.forward(cfg, xt, idt, twt, wd, again, ws)      # run to run: bit-identical
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    return dict(x=x, wr=wr, b=b, ids=idt.cpu().numpy(), tw=twt.cpu().numpy(),
                out=out.view(torch.int16).cpu().numpy().view(np.uint16))


def _oracle(w, r, tokens=None, edge=False, gain=1.0, **kw):
    return L.moe_layer(oracle_cfg(w, **kw), r["x"], r["wr"], r["b"], ExpertSource(w, gain, edge), tokens=tokens,
                       topk_ids=r["ids"], topk_w=r["tw"], workers=ORACLE_WORKERS)["out"]


@pytest.mark.parametrize("key", ["decode_nvfp4", "decode_mxfp8"])
def test_inkling_decode_every_token(gpu_lib, key):
    """The decode batches (64 NVFP4 / 192 MXFP8 tokens, 384 experts): every
    token's output against the oracle."""
    w = synth.WORKLOADS[key]
    r = _run(gpu_lib, w)
    assert rel_err(r["out"], _oracle(w, r)) <= OUT_RTOL


def test_inkling_ep_share_every_token(gpu_lib):
    """The EP8 share (4096 tokens, experts 0-47 local, 128-row MXFP8 tiles):
    every token with a local pair against the oracle; tokens without one
    have an exactly zero partial sum."""
    w = synth.WORKLOADS["ep8_mxfp8"]
    r = _run(gpu_lib, w)
    loc = (r["ids"] >= w.expert_begin) & (r["ids"] < w.expert_begin + w.num_local)
    toks = np.nonzero(loc.any(1))[0]
    assert np.all(r["out"][~loc.any(1)] & 0x7FFF == 0)
    assert rel_err(r["out"][toks], _oracle(w, r, tokens=toks)) <= OUT_RTOL


def test_inkling_prefill_every_row_of_the_hottest_experts(gpu_lib):
    """The 16384-token NVFP4 prefill chunk (Zipf bias) with its full router,
    computed for a local set of 4 experts that includes the most loaded one
    (thousands of rows: every row position of the 128-row tiles, full and
    partial): every token with a local pair against the oracle."""
    w = synth.WORKLOADS["prefill_nvfp4"]
    _, _, _, ids, _, _ = _run_route(gpu_lib, w)
    hot = int(np.bincount(ids.ravel(), minlength=w.experts).argmax())
    begin = min(max(hot - 1, 0), w.experts - 4)
    wl = synth.Workload("prefill_local4", w.name, w.tokens, w.hidden, w.experts, w.top_k, w.ffn, w.fmt, w.seed,
                        bias=w.bias, expert_begin=begin, num_local=4)
    r = _run(gpu_lib, wl)
    assert np.array_equal(r["ids"], ids)
    loc = (ids >= begin) & (ids < begin + 4)
    counts = np.bincount(ids[loc] - begin, minlength=4)
    assert counts.max() > 1024 and np.any(counts % 128 != 0)
    toks = np.nonzero(loc.any(1))[0]
    assert np.all(r["out"][~loc.any(1)] & 0x7FFF == 0)
    assert rel_err(r["out"][toks], _oracle(wl, r, tokens=toks)) <= OUT_RTOL


# --------------------------------------------------- edge-case activations --

def _edge_tokens(T, H, seed):
    """bf16 rows by class: 0 normal N(0,1); 1 zero; 2 negative zero; 3 every
    other 16-block x 1e-5 (subnormal E4M3 block scales); 4 every other block
    x 1e-8 (zero block scales); 5 huge (x 2^60); 6 tiny (x 2^-40, so that
    the SwiGLU output, quadratic in x, stays in fp32's normal range); 7 half
    the row zero."""
    g = np.random.default_rng(seed)
    v = g.standard_normal((T, H)).astype(np.float32)
    cls = np.arange(T) % 8
    blk = (np.arange(H) // 16) % 2 == 1
    v[cls == 1] = 0.0
    v[cls == 2] = -0.0
    v[np.ix_(cls == 3, blk)] *= np.float32(1e-5)
    v[np.ix_(cls == 4, blk)] *= np.float32(1e-8)
    v[cls == 5] *= np.float32(2.0 ** 60)
    v[cls == 6] *= np.float32(2.0 ** -40)
    v[cls == 7, H // 2:] = 0.0
    return synth.to_bf16_bits(v), cls


EDGE_X = {   # keyed by format and rows per work-list entry
    "nvfp4_32": synth.Workload("ex1", "edge x", 96, 512, 32, 4, 256, "nvfp4", 61, weights="gaussian"),
    "mxfp8_32": synth.Workload("ex2", "edge x", 96, 512, 32, 4, 256, "mxfp8", 62, weights="gaussian"),
    "nvfp4_128": synth.Workload("ex3", "edge x", 2048, 256, 16, 2, 128, "nvfp4", 63, weights="gaussian"),
    "mxfp8_128": synth.Workload("ex4", "edge x", 2048, 256, 16, 2, 128, "mxfp8", 64, weights="gaussian"),
}


@pytest.mark.parametrize("cap_form", [0, 3])
@pytest.mark.parametrize("key", list(EDGE_X))
def test_edge_case_activations(gpu_lib, key, cap_form):
    """Zero, -0, huge, tiny, half-zero rows and rows whose NVFP4 blocks get
    subnormal or zero block scales, through route + forward (32-row and
    128-row work-list entries).  Each row class is held to the bar against
    its own maximum; zero rows give exactly zero.

    Huge rows are checked with the cap off (cap_form 3) only: under a cap
    they saturate it, and h then jumps from about -0.006 c to 0.99 c^2 as g
    crosses zero, while g's absolute rounding error from any fp32
    accumulation grows with x (about 10 at x ~ 2^24); an element whose g
    falls near zero then differs by a whole jump whatever the summation
    order.  Without the cap, h = silu(g) u is continuous there."""
    import torch
    w = EDGE_X[key]
    bse = gpu_lib
    x, cls = _edge_tokens(w.tokens, w.hidden, w.seed)
    wr = synth.router_weight(w.seed, w.experts, w.hidden)
    b = synth.router_bias(w.seed, w.experts)
    cfg = lib_cfg(bse, w, cap_form=cap_form)
    stacked, ews = stack_local(w)
    wd = bse.prepare_weights(cfg, {kk: to_dev(v) for kk, v in stacked.items()})
    ws = bse.workspace(cfg)
    T = w.tokens
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    xt = to_dev(x.view(np.int16), torch.bfloat16)
    out = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
    bse.route(cfg, xt, to_dev(wr.view(np.int16), torch.bfloat16), to_dev(b), ids, tw, None, ws)
    bse.forward(cfg, xt, ids, tw, wd, out, ws)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = L.moe_layer(oracle_cfg(w, cap_form=cap_form), x, wr, b, ews, topk_ids=ids.cpu().numpy(),
                      topk_w=tw.cpu().numpy())["out"]
    for c in range(8):
        rows = cls == c
        if c == 5 and cap_form != 3:
            continue
        if c in (1, 2):
            assert np.all(bf16_to_f64(got[rows]) == 0) and np.all(bf16_to_f64(ref[rows]) == 0)
        else:
            assert rel_err(got[rows], ref[rows]) <= OUT_RTOL, c


# ------------------------------------------------------ edge-case weights --

@pytest.mark.parametrize("T", [64, 2400])
@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_edge_case_weights_inkling_size(gpu_lib, fmt, kind, T):
    """One Inkling-size expert drawn with zero and subnormal block scales
    (NVFP4) or zero and subnormal elements over the whole exponent range
    (MXFP8), see synth; every token routed to it in slot 0 (64 tokens: 16-row
    entries of the decode kernel; 2400: 128-row entries of the large-M
    kernels), the other slots pointing at experts that are not local."""
    E, k = 384, 8
    e = 30 + kind
    w = synth.Workload("edge_w", "edge weights", T, 4608, E, k, 2304, fmt, 70 + kind, expert_begin=e, num_local=1)
    g = np.random.default_rng(T + kind)
    others = np.array([i for i in range(E) if i != e])
    ids = np.stack([np.concatenate([[e], g.choice(others, k - 1, replace=False)]) for _ in range(T)]).astype(np.int32)
    tw = g.uniform(0.05, 0.3, size=(T, k)).astype(np.float32)
    r = _run(gpu_lib, w, ids=ids, tw=tw, edge=True)
    ref = _oracle(w, r, edge=True)
    assert np.abs(bf16_to_f64(ref)).max() > 0
    assert rel_err(r["out"], ref) <= OUT_RTOL
