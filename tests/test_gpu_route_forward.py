"""moe_route_forward on the GPU: for small batches routing, x quantization
and dispatch run as one launch, whose results must be bit-identical to
moe_route + moe_forward (the same router, quantizer and dispatch bodies),
and held to the oracle's bars: routing sets exact away from near ties,
the layer output within 2e-2 (max-abs normalised, routing replayed).

Shapes cover every router variant of the one launch (16 / 32 / 64-token
GEMV tiles, 6 / 4 / 2 K slices, top-k widths 1 to 16 experts per lane),
both formats, static NVFP4 activation scales, EP shares, repeated calls on
one workspace (the completion flags of earlier calls must never satisfy a
later call's waits), and batches above 256 tokens or 4096 pairs (the launch
sequence of moe_route and moe_forward).
"""
import numpy as np
import pytest

import synth
from oracle import layer as L

from _util import ORACLE_WORKERS, OUT_RTOL, ExpertSource, inputs, lib_cfg, oracle_cfg, rel_err, stack_local, to_dev
from test_gpu_route_dispatch import _check_route

pytestmark = pytest.mark.gpu


class Layer:
    """Weights of workload w in HBM (packed) and a workspace for up to
    max_tokens tokens; runs both entry points on the first T tokens."""

    def __init__(self, bse, w, max_tokens, **kw):
        import torch
        self.bse, self.w = bse, w
        self.cfg = lib_cfg(bse, w, max_tokens=max_tokens, **kw)
        stacked, self.ews = stack_local(w)
        self.wd = bse.prepare_weights(self.cfg, {k: to_dev(v) for k, v in stacked.items()})
        self.ws = bse.workspace(self.cfg)
        self.x, self.wr, self.b = inputs(w, max_tokens)
        self.xt = to_dev(self.x.view(np.int16), torch.bfloat16)
        self.wrt, self.bt = to_dev(self.wr.view(np.int16), torch.bfloat16), to_dev(self.b)

    def run(self, T, one_call):
        import torch
        w = self.w
        ids = torch.full((T, w.top_k), -5, dtype=torch.int32, device="cuda")
        tw = torch.full((T, w.top_k), -5.0, dtype=torch.float32, device="cuda")
        nt = torch.full((T,), 7, dtype=torch.uint8, device="cuda")
        out = torch.full((T, w.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        x = self.xt[:T]
        if one_call:
            self.bse.route_forward(self.cfg, x, self.wrt, self.bt, ids, tw, nt, self.wd, out, self.ws)
        else:
            self.bse.route(self.cfg, x, self.wrt, self.bt, ids, tw, nt, self.ws)
            self.bse.forward(self.cfg, x, ids, tw, self.wd, out, self.ws)
        torch.cuda.synchronize()
        return dict(ids=ids.cpu().numpy(), tw=tw.cpu().numpy(), nt=nt.cpu().numpy().astype(bool),
                    out=out.view(torch.int16).cpu().numpy().view(np.uint16))


def _same(a, b):
    for key in ("ids", "tw", "nt", "out"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


@pytest.fixture(scope="module")
def inkling_nvfp4(gpu_lib):
    return Layer(gpu_lib, synth.WORKLOADS["decode_nvfp4"], 300)


@pytest.mark.parametrize("T", [1, 4, 16, 17, 32, 33, 64, 100, 129, 256, 257, 300])
def test_inkling_nvfp4_bit_identical_to_route_then_forward(inkling_nvfp4, T):
    a = inkling_nvfp4.run(T, one_call=True)
    b = inkling_nvfp4.run(T, one_call=False)
    _same(a, b)


@pytest.mark.parametrize("T", [1, 4, 16, 32])
def test_inkling_nvfp4_small_batches_vs_oracle(inkling_nvfp4, T):
    """Small decode batches through the one launch, every token against the
    oracle: routing sets and order, gate weights, and the layer output."""
    lay = inkling_nvfp4
    w = lay.w
    r = lay.run(T, one_call=True)
    x = lay.x[:T]
    _check_route(w, x, lay.wr, lay.b, r["ids"], r["tw"], r["nt"])
    ref = L.moe_layer(oracle_cfg(w), x, lay.wr, lay.b, ExpertSource(w), topk_ids=r["ids"], topk_w=r["tw"],
                      workers=ORACLE_WORKERS)["out"]
    assert rel_err(r["out"], ref) <= OUT_RTOL


def test_repeated_calls_on_one_workspace(inkling_nvfp4):
    """Batches of different sizes in turn on one workspace: every call's
    waits see only its own completion flags."""
    ref = {T: inkling_nvfp4.run(T, one_call=False) for T in (64, 3, 200)}
    for T in (64, 3, 200, 3, 64, 200):
        _same(inkling_nvfp4.run(T, one_call=True), ref[T])


SHAPES = {
    # (workload, T values): every top-k width and token-tile height
    "e40_mxfp8": (synth.Workload("rf1", "rf", 256, 256, 40, 4, 128, "mxfp8", 81, weights="gaussian"), (1, 20, 40, 256)),
    "e100_nvfp4": (synth.Workload("rf2", "rf", 200, 512, 100, 6, 256, "nvfp4", 82, weights="gaussian"), (5, 30, 70, 200)),
    "e200_mxfp8": (synth.Workload("rf3", "rf", 130, 256, 200, 8, 128, "mxfp8", 83, weights="gaussian"), (2, 64, 130)),
    "e600_nvfp4": (synth.Workload("rf4", "rf", 100, 256, 600, 8, 128, "nvfp4", 84, weights="gaussian"), (9, 100)),
    "ep_share": (synth.Workload("rf5", "rf", 150, 512, 32, 4, 256, "mxfp8", 85, weights="gaussian",
                                expert_begin=8, num_local=8), (1, 33, 150)),
    # top-20 of 64: 200 tokens are 4000 pairs (one launch), 256 are 5120 (the launch sequence)
    "top20": (synth.Workload("rf6", "rf", 256, 256, 64, 20, 128, "nvfp4", 86, weights="gaussian"), (200, 256)),
}


@pytest.mark.parametrize("key", list(SHAPES))
def test_shapes_bit_identical_and_vs_oracle(gpu_lib, key):
    w, Ts = SHAPES[key]
    lay = Layer(gpu_lib, w, max(Ts))
    for T in Ts:
        a = lay.run(T, one_call=True)
        _same(a, lay.run(T, one_call=False))
        _check_route(w, lay.x[:T], lay.wr, lay.b, a["ids"], a["tw"], a["nt"])
        ref = L.moe_layer(oracle_cfg(w), lay.x[:T], lay.wr, lay.b, lay.ews, topk_ids=a["ids"], topk_w=a["tw"])["out"]
        assert rel_err(a["out"], ref) <= OUT_RTOL, (key, T)


def test_static_nvfp4_activation_scales(gpu_lib):
    w = synth.Workload("rf7", "rf", 64, 512, 32, 4, 256, "nvfp4", 87, weights="gaussian")
    act = (2, (4.0 / 2688, 0.25 / 2688))
    lay = Layer(gpu_lib, w, 64, act_gs=act[0], act_gs_static=act[1])
    a = lay.run(64, one_call=True)
    _same(a, lay.run(64, one_call=False))
    ref = L.moe_layer(oracle_cfg(w, act_gs="static", act_gs_static=tuple(np.float32(v) for v in act[1])),
                      lay.x, lay.wr, lay.b, lay.ews, topk_ids=a["ids"], topk_w=a["tw"])["out"]
    assert rel_err(a["out"], ref) <= OUT_RTOL
