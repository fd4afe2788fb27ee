"""moe_forward_fused (the expert half in one launch) on the GPU.

Its work items run the same tile bodies, the same h quantization and the
same fixed-order combine as moe_forward's launch sequence, so the two
outputs must be bit-identical; each is also held to the oracle's bar
(max|gpu - oracle| / max|oracle| <= 2e-2, routing replayed).  Shapes cover
all three work-list entry heights the single launch serves (16, 32 and
64 rows), both formats and weight layouts, EP shares (partial sums), a
single token, Inkling-size decode batches, repeated calls on one workspace
(the control words are cleared by each call's dispatch launch) and batches
outside its range (128-row entries, more than 4096 pairs: moe_forward's
launch sequence runs).
"""
import numpy as np
import pytest

import synth

from _util import OUT_RTOL, rel_err
from test_gpu_forward import SMALL, oracle_out, run_layer

pytestmark = pytest.mark.gpu

CASES = {
    # expected rows per local expert <= 2: 16-row entries
    "tiny": synth.WORKLOADS["tiny"],
    # 4..24: 32-row entries
    "mid_nvfp4": SMALL["mid_nvfp4"],
    "mid_mxfp8": SMALL["mid_mxfp8"],
    "ep_nvfp4": SMALL["ep_nvfp4"],
    "ep_mxfp8": SMALL["ep_mxfp8"],
    # 24..48: 64-row entries
    "rows64_nvfp4": synth.Workload("rows64_nvfp4", "64-row entries", 256, 512, 32, 4, 256, "nvfp4", 41,
                                   weights="gaussian"),
    "rows64_mxfp8": synth.Workload("rows64_mxfp8", "64-row entries", 240, 256, 24, 4, 256, "mxfp8", 42,
                                   weights="gaussian"),
    # skewed loads: many experts with one entry, a few with several
    "zipf_nvfp4": synth.Workload("zipf_nvfp4", "skewed", 96, 512, 64, 6, 256, "nvfp4", 43, bias="zipf",
                                 weights="gaussian"),
    # 128-row entries: outside the single launch's range
    "many_rows": SMALL["many_rows"],
    # more than 4096 pairs with 64-row entries: outside its range too (the
    # general dispatch runs, then moe_forward's launch sequence)
    "pairs_over_4096": synth.Workload("pairs_over_4096", "general dispatch", 600, 256, 128, 8, 128, "nvfp4", 44,
                                      weights="gaussian"),
}


@pytest.mark.parametrize("key", list(CASES))
def test_fused_matches_launch_sequence_and_oracle(gpu_lib, key):
    w = CASES[key]
    a = run_layer(gpu_lib, w)
    b = run_layer(gpu_lib, w, fused=True)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["out"], b["out"])
    assert rel_err(b["out"], oracle_out(w, b)) <= OUT_RTOL


@pytest.mark.parametrize("layout", ["canonical", "packed"])
def test_fused_single_token(gpu_lib, layout):
    w = SMALL["mid_mxfp8"]
    a = run_layer(gpu_lib, w, T=1, max_tokens=200, layout=layout)
    b = run_layer(gpu_lib, w, T=1, max_tokens=200, layout=layout, fused=True)
    assert np.array_equal(a["out"], b["out"])
    assert rel_err(b["out"], oracle_out(w, b)) <= OUT_RTOL


@pytest.mark.parametrize("key", ["decode_nvfp4", "decode_mxfp8"])
def test_fused_inkling_decode_bit_exact(gpu_lib, key):
    """Inkling-size decode batches: bit-identical to moe_forward on every
    token, and sampled tokens against the oracle."""
    w = synth.WORKLOADS[key]
    a = run_layer(gpu_lib, w)
    b = run_layer(gpu_lib, w, fused=True)
    assert np.array_equal(a["out"], b["out"])
    b["ews"] = None
    toks = np.random.default_rng(2).choice(w.tokens, 2, replace=False)
    assert rel_err(b["out"][toks], oracle_out(w, b, tokens=toks)) <= OUT_RTOL


def test_fused_repeated_calls_one_workspace(gpu_lib):
    """Several calls on one workspace, with batches of different sizes: each
    call's dispatch launch clears the queue and counters the last one left."""
    import torch
    from _util import inputs, lib_cfg, stack_local, to_dev
    bse = gpu_lib
    w = SMALL["mid_nvfp4"]
    cfg = lib_cfg(bse, w, max_tokens=w.tokens)
    stacked, _ = stack_local(w)
    wd = bse.prepare_weights(cfg, {k: to_dev(v) for k, v in stacked.items()})
    ws = bse.workspace(cfg)
    x, wr, b = inputs(w, w.tokens)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wrt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(b).cuda()
    for T in (w.tokens, 7, w.tokens, 1, 33):
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
        ref = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
        out = torch.empty_like(ref)
        bse.route(cfg, xt[:T], wrt, bt, ids, tw, None, ws)
        bse.forward(cfg, xt[:T], ids, tw, wd, ref, ws)
        bse.forward(cfg, xt[:T], ids, tw, wd, out, ws, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), T


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_fused_cap_forms_under_stress(gpu_lib, form, fmt):
    """Expert weights x10 so gate/up values pass the cap: every capped-SwiGLU
    form in the single launch's gate/up items."""
    w = synth.Workload("cap", "cap stress", 48, 512, 16, 4, 256, fmt, 27, weights="gaussian")
    a = run_layer(gpu_lib, w, gain=10.0, cap_form=form)
    b = run_layer(gpu_lib, w, gain=10.0, cap_form=form, fused=True)
    assert np.array_equal(a["out"], b["out"])
    assert rel_err(b["out"], oracle_out(w, b, cap_form=form)) <= OUT_RTOL


@pytest.mark.parametrize("mode", [1, 2])
def test_fused_with_shared_activation_scales_runs_the_sequence(gpu_lib, mode):
    """Per-tensor and static NVFP4 activation scales: moe_forward_fused runs
    moe_forward's launch sequence (bit-identical) and reports status 0."""
    w = CASES["mid_nvfp4"]
    act = (mode, (4.0 / 2688, 0.25 / 2688))
    a = run_layer(gpu_lib, w, act=act)
    b = run_layer(gpu_lib, w, act=act, fused=True)
    assert np.array_equal(a["out"], b["out"]) and b["fused_err"] == 0


def test_fused_error_word_poisons_the_output(gpu_lib, monkeypatch):
    """The failure path of the bounded waits, forced from the host: with
    MOE_FUSED_TEST_FAIL=1 the launch starts with its error word set, every
    wait returns at once, the launch drains, every combine item writes bf16
    NaN, and moe_forward_fused_status reports 1.  A later call without the
    hook is clean again."""
    w = CASES["mid_nvfp4"]
    monkeypatch.setenv("MOE_FUSED_TEST_FAIL", "1")
    bad = run_layer(gpu_lib, w, fused=True, expect_fused_err=1)
    assert np.all(bad["out"] == 0x7FC0)
    monkeypatch.delenv("MOE_FUSED_TEST_FAIL")
    good = run_layer(gpu_lib, w, fused=True)
    ref = run_layer(gpu_lib, w)
    assert np.array_equal(good["out"], ref["out"])
