"""moe_route + moe_forward on the GPU vs the oracle's whole layer.

The bf16 output must satisfy max|gpu - oracle| / max|oracle| <= 2e-2.  The
oracle is run with the GPU's routing replayed (so near ties cannot make the
two sides pick different experts); routing itself is checked in
test_gpu_route_dispatch.py.  Small shapes are checked on every token; the
Inkling-size workloads on sampled tokens the oracle computes one by one.
"""
import numpy as np
import pytest

import synth
from oracle import layer as L

from _util import OUT_RTOL, inputs, lib_cfg, oracle_cfg, rel_err, stack_local, to_dev, expert_weights

pytestmark = pytest.mark.gpu


def run_layer(bse, w, gain=1.0, T=None, cap_form=None, max_tokens=None, layout="packed", fused=False, act=None,
              expect_fused_err=0, x=None, ids=None, tw=None):
    """act: optional (act_gs mode, (x scale, h scale)) for NVFP4 activations.
    fused: moe_forward_fused, whose status word must equal expect_fused_err.
    x: optional bf16 token rows (bits) in place of the workload's.
    ids, tw: optional routing to replay (moe_route is then not called)."""
    import torch
    x0, wr, b = inputs(w, T)
    x = x0 if x is None else x
    T = x.shape[0]
    kw = {} if cap_form is None else {"cap_form": cap_form}
    if act is not None:
        kw.update(act_gs=act[0], act_gs_static=act[1])
    cfg = lib_cfg(bse, w, max_tokens=max_tokens or T, **kw)
    stacked, ews = stack_local(w, gain)
    wd = {k: to_dev(v) for k, v in stacked.items()}
    if layout == "packed":
        wd = bse.prepare_weights(cfg, wd)
    ws = bse.workspace(cfg)
    replay = ids is not None
    if replay:
        ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
        tw = torch.from_numpy(np.ascontiguousarray(tw, dtype=np.float32)).cuda()
    else:
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    nt = torch.empty(T, dtype=torch.uint8, device="cuda")
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wrt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
    if not replay:
        bse.route(cfg, xt, wrt, torch.from_numpy(b).cuda(), ids, tw, nt, ws)
    bse.forward(cfg, xt, ids, tw, wd, out, ws, fused=fused)
    fused_err = None
    if fused:   # the single launch's error word: every dependency wait met
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        bse.forward_fused_status(cfg, T, ws, err)
        fused_err = int(err.cpu().item())
        assert fused_err == expect_fused_err
    torch.cuda.synchronize()
    return dict(x=x, wr=wr, b=b, ids=ids.cpu().numpy(), tw=tw.cpu().numpy(),
                out=out.view(torch.int16).cpu().numpy().view(np.uint16), ews=ews, fused_err=fused_err)


ACT_NAMES = {0: "row", 1: "tensor", 2: "static"}


def oracle_out(w, r, tokens=None, gain=1.0, cap_form=None, act=None):
    kw = {} if cap_form is None else {"cap_form": cap_form}
    if act is not None:
        kw.update(act_gs=ACT_NAMES[act[0]], act_gs_static=tuple(np.float32(v) for v in act[1]))
    cfg = oracle_cfg(w, **kw)
    if r.get("ews") is not None:
        ew = r["ews"]
    else:
        ew = lambda e: expert_weights(w, e, gain)  # noqa: E731
    res = L.moe_layer(cfg, r["x"], r["wr"], r["b"], ew, tokens=tokens, topk_ids=r["ids"], topk_w=r["tw"])
    return res["out"]


@pytest.mark.parametrize("key", ["tiny"])
def test_tiny_layer_all_tokens(gpu_lib, key):
    w = synth.WORKLOADS[key]
    r = run_layer(gpu_lib, w)
    ref = oracle_out(w, r)
    assert rel_err(r["out"], ref) <= OUT_RTOL


SMALL = {
    "mid_nvfp4": synth.Workload("mid_nvfp4", "mid NVFP4", 100, 1024, 32, 4, 512, "nvfp4", 21, weights="gaussian"),
    "mid_mxfp8": synth.Workload("mid_mxfp8", "mid MXFP8", 77, 512, 24, 3, 384, "mxfp8", 22, weights="gaussian"),
    "ep_mxfp8": synth.Workload("ep_mxfp8", "EP share", 150, 512, 32, 4, 256, "mxfp8", 23, weights="gaussian",
                               expert_begin=8, num_local=8),
    "ep_nvfp4": synth.Workload("ep_nvfp4", "EP share", 130, 512, 32, 4, 256, "nvfp4", 24, weights="gaussian",
                               expert_begin=20, num_local=12),
    "many_rows": synth.Workload("many_rows", "rows > tile", 700, 256, 8, 2, 128, "nvfp4", 25, weights="gaussian"),
    "many_rows8": synth.Workload("many_rows8", "rows > tile", 700, 256, 8, 2, 128, "mxfp8", 26, weights="gaussian"),
}


@pytest.mark.parametrize("key", list(SMALL))
def test_small_layers_all_tokens(gpu_lib, key):
    w = SMALL[key]
    r = run_layer(gpu_lib, w)
    ref = oracle_out(w, r)
    assert rel_err(r["out"], ref) <= OUT_RTOL


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_cap_forms_under_stress(gpu_lib, form, fmt):
    """Expert weights x10 so gate/up values pass the cap (7.0)."""
    w = synth.Workload("cap", "cap stress", 48, 512, 16, 4, 256, fmt, 27, weights="gaussian")
    r = run_layer(gpu_lib, w, gain=10.0, cap_form=form)
    ref = oracle_out(w, r, cap_form=form)
    assert rel_err(r["out"], ref) <= OUT_RTOL


# Skewed expert loads (Zipf bias) over 48 experts at about 170 rows each: the
# experts' last 128-row tiles hold every count of 16-row sub-tiles from 1 to 8
# (the large-M kernels compile one tile body per count).
RAGGED = {
    "nvfp4": synth.Workload("ragged_nvfp4", "ragged last tiles", 2048, 256, 48, 4, 128, "nvfp4", 28,
                            bias="zipf", weights="gaussian"),
    "nvfp4_wide": synth.Workload("ragged_nvfp4_wide", "ragged last tiles", 2048, 512, 48, 4, 256, "nvfp4", 30,
                                 bias="zipf", weights="gaussian"),
    "mxfp8": synth.Workload("ragged_mxfp8", "ragged last tiles", 2048, 256, 48, 4, 128, "mxfp8", 29,
                            bias="zipf", weights="gaussian"),
}


@pytest.mark.parametrize("fmt", list(RAGGED))
def test_large_m_partial_tiles_every_subtile_count(gpu_lib, fmt):
    w = RAGGED[fmt]
    r = run_layer(gpu_lib, w)
    rem = np.bincount(r["ids"].ravel(), minlength=w.experts) % 128
    assert set(int(v) for v in np.ceil(rem[rem > 0] / 16)) == set(range(1, 9))
    assert rel_err(r["out"], oracle_out(w, r)) <= OUT_RTOL


# Per-row activation scales and per-row GEMM arithmetic: a token's output
# does not depend on the other tokens of the batch.  At one batch size (so
# the same kernels and tile heights) replacing two of every three tokens
# leaves the kept tokens' rows bit-identical, although the dispatch places
# them at other positions of other tiles.
@pytest.mark.parametrize("key", ["decode_nvfp4", "ragged_mxfp8", "ragged_nvfp4"])
def test_token_rows_independent_of_the_rest_of_the_batch(gpu_lib, key):
    ragged = {w.key: w for w in RAGGED.values()}
    w = ragged.get(key) or synth.WORKLOADS[key]
    a = run_layer(gpu_lib, w)
    x2 = a["x"].copy()
    other = np.arange(w.tokens) % 3 != 0
    x2[other] = synth.tokens(w.seed + 1000, w.tokens, w.hidden)[other]
    b = run_layer(gpu_lib, w, x=x2)
    kept = ~other
    assert np.array_equal(a["ids"][kept], b["ids"][kept])
    assert not np.array_equal(a["ids"][other], b["ids"][other])
    assert np.array_equal(a["out"][kept], b["out"][kept])


def _bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("key", ["mid_nvfp4", "mid_mxfp8"])
def test_topk_slot_permutation_changes_only_the_combine_rounding(gpu_lib, key):
    """Replaying the routing with each token's k slots permuted: every pair's
    expert output is the same, and the combine sums the same products in
    another fp32 order, so each output element moves by at most one bf16 step
    (plus fp32 reordering error where terms cancel), and the oracle bar
    holds."""
    w = SMALL[key]
    a = run_layer(gpu_lib, w)
    g = np.random.default_rng(9)
    perm = np.stack([g.permutation(w.top_k) for _ in range(w.tokens)])
    b = run_layer(gpu_lib, w, ids=np.take_along_axis(a["ids"], perm, 1), tw=np.take_along_axis(a["tw"], perm, 1))
    fa, fb = _bf16_f64(a["out"]), _bf16_f64(b["out"])
    # one bf16 step of the larger value, plus a small absolute slack for
    # elements whose terms cancel (fp32 reordering error of the products)
    bound = np.maximum(np.abs(fa), np.abs(fb)) * 2.0 ** -7 + np.abs(fa).max() * 2.0 ** -16
    assert np.all(np.abs(fa - fb) <= bound)
    assert not np.array_equal(a["ids"], b["ids"])
    assert rel_err(b["out"], oracle_out(w, b)) <= OUT_RTOL


def test_single_token_and_max_tokens_margin(gpu_lib):
    w = SMALL["mid_nvfp4"]
    r = run_layer(gpu_lib, w, T=1, max_tokens=300)
    assert rel_err(r["out"], oracle_out(w, r)) <= OUT_RTOL


# The decode batches and the EP share are compared on every token in
# test_gpu_parity_full.py; the whole prefill chunk (whose y exceeds the
# last-level cache and streams) on sampled tokens here.
@pytest.mark.parametrize("key,ntok", [("prefill_nvfp4", 2)])
def test_inkling_workloads_sampled(gpu_lib, key, ntok):
    w = synth.WORKLOADS[key]
    r = run_layer(gpu_lib, w)
    r["ews"] = None
    rng = np.random.default_rng(1)
    if w.num_local is not None:   # tokens with at least one local expert
        loc = (r["ids"] >= w.expert_begin) & (r["ids"] < w.expert_begin + w.num_local)
        toks = rng.choice(np.nonzero(loc.any(1))[0], ntok, replace=False)
    else:
        toks = rng.choice(w.tokens, ntok, replace=False)
    ref = oracle_out(w, r, tokens=toks)
    assert rel_err(r["out"][toks], ref) <= OUT_RTOL
    # determinism: a second run is bit-identical
    r2 = run_layer(gpu_lib, w)
    assert np.array_equal(r2["out"], r["out"])


@pytest.mark.parametrize("key", ["tiny", "mid_nvfp4", "mid_mxfp8", "ep_nvfp4", "ragged_nvfp4", "ragged_nvfp4_wide",
                                 "ragged_mxfp8", "decode_nvfp4", "decode_mxfp8"])
def test_packed_layout_matches_canonical_bit_exact(gpu_lib, key):
    """moe_prepare_weights only permutes bytes: the layer output with packed
    weights is bit-identical to the output with the canonical arrays."""
    ragged = {w.key: w for w in RAGGED.values()}
    w = SMALL.get(key) or ragged.get(key) or synth.WORKLOADS[key]
    a = run_layer(gpu_lib, w, layout="canonical")
    b = run_layer(gpu_lib, w, layout="packed")
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["out"], b["out"])


# NVFP4 activation scales per tensor and static (the alternatives of the
# per-row reading): the one-launch quantize + dispatch (<= 4096 pairs, 32-row
# entries), the large-M kernels (128-row entries) and the general dispatch
# (more than 4096 pairs), every token against the oracle.
ACT_CASES = {
    "mid_nvfp4": SMALL["mid_nvfp4"],
    "many_rows": SMALL["many_rows"],
    "pairs_over_4096": synth.Workload("pairs_over_4096", "general dispatch", 600, 256, 128, 8, 128, "nvfp4", 44,
                                      weights="gaussian"),
}


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("key", list(ACT_CASES))
def test_nvfp4_shared_activation_scales(gpu_lib, key, mode):
    w = ACT_CASES[key]
    act = (mode, (4.0 / 2688, 0.25 / 2688))
    r = run_layer(gpu_lib, w, act=act)
    ref = oracle_out(w, r, act=act)
    assert rel_err(r["out"], ref) <= OUT_RTOL
    # the shared scales change the result (they are not the per-row ones)
    assert not np.array_equal(ref, oracle_out(w, r))
