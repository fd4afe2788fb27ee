"""Pins against the numbers the pages print (tests/golden/pages_constants.json).

The pages print no worked numeric example of the layer, but they do print
the model's size and the size of both checkpoints.  Those pin the shapes and
the byte layout of the two block formats the oracle encodes: the expert byte
count that the oracle's own encoder produces, times 384 experts and the
per-layer format map, plus the non-expert parameters in BF16, must land on
the printed checkpoint sizes, and the alternatives (a 32-element NVFP4
block, an E8M0 NVFP4 block scale, a wider FFN) must not.
"""
import json
import os

import numpy as np
import pytest

from oracle import layer as L

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def v(key):
    return GOLD[key]["value"]


def _expert_bytes_from_encoder(fmt, H, Fd):
    z = np.zeros((Fd, H), dtype=np.float32)
    zd = np.zeros((H, Fd), dtype=np.float32)
    ew = L.quantize_expert_weights(fmt, z, z, zd)
    return sum(np.asarray(a).nbytes for a in ew.values())


@pytest.fixture(scope="module")
def expert_bytes():
    H, Fd = v("hidden"), v("moe_ffn")
    return {fmt: _expert_bytes_from_encoder(fmt, H, Fd) for fmt in ("nvfp4", "mxfp8")}


def test_parameter_counts():
    H, Fd, E, k, nl = v("hidden"), v("moe_ffn"), v("experts"), v("top_k"), v("layers")
    per_expert = 3 * H * Fd                      # gate, up, down of a SwiGLU expert
    expert_params = nl * E * per_expert
    rest = v("total_params_B") * 1e9 - expert_params
    assert 0 < rest < 0.02 * v("total_params_B") * 1e9
    active = nl * k * per_expert + rest          # no shared experts
    assert abs(active / 1e9 - v("active_params_B")[1]) < 0.5     # "about 19B"


def test_expert_bytes(expert_bytes):
    assert expert_bytes["nvfp4"] == 17_915_916
    assert expert_bytes["mxfp8"] == 32_845_824


def _ckpt_gb(bytes_nv, bytes_mx):
    H, Fd, E, nl = v("hidden"), v("moe_ffn"), v("experts"), v("layers")
    lo, hi = v("nvfp4_layers")
    n_nv = hi - lo + 1
    n_mx = nl - n_nv
    rest_params = v("total_params_B") * 1e9 - nl * E * 3 * H * Fd
    rest_bytes = 2 * rest_params                 # "the rest BF16"
    mixed = (n_nv * E * bytes_nv + n_mx * E * bytes_mx + rest_bytes) / 1e9
    allmx = (nl * E * bytes_mx + rest_bytes) / 1e9
    return mixed, allmx


def _experts_gb(bytes_nv, bytes_mx):
    E, nl = v("experts"), v("layers")
    lo, hi = v("nvfp4_layers")
    n_nv = hi - lo + 1
    return (n_nv * E * bytes_nv + (nl - n_nv) * E * bytes_mx) / 1e9, nl * E * bytes_mx / 1e9


def test_checkpoint_sizes_pin_block_formats(expert_bytes):
    mixed, allmx = _ckpt_gb(expert_bytes["nvfp4"], expert_bytes["mxfp8"])
    assert abs(mixed / v("ckpt_mixed_GB") - 1) < 0.02
    assert abs(allmx / v("ckpt_mxfp8_GB") - 1) < 0.02
    # the per-GPU figures at TP4 / EP4 are the routed experts split four ways
    ex_mixed, ex_mx = _experts_gb(expert_bytes["nvfp4"], expert_bytes["mxfp8"])
    assert abs(ex_mixed / 4 / v("per_gpu_tp4_mixed_GB") - 1) < 0.01
    assert abs(ex_mx / 4 / v("per_gpu_tp4_mxfp8_GB") - 1) < 0.01
    # at TP2 the whole checkpoint is split two ways
    assert abs(allmx / 2 / v("per_gpu_tp2_mxfp8_GB") - 1) < 0.01


def test_alternative_layouts_miss_the_printed_sizes(expert_bytes):
    H, Fd = v("hidden"), v("moe_ffn")
    n = 3 * H * Fd
    alternatives = {
        "fp4 with one byte scale per 32": n // 2 + n // 32 + 12,
        "fp4 without block scales": n // 2 + 12,
        "fp6-like 6-bit elements per 16": 3 * n // 4 + n // 16 + 12,
    }
    for name, nb in alternatives.items():
        mixed, _ = _ckpt_gb(nb, expert_bytes["mxfp8"])
        ex_mixed, _ = _experts_gb(nb, expert_bytes["mxfp8"])
        assert abs(mixed / v("ckpt_mixed_GB") - 1) > 0.04, name
        assert abs(ex_mixed / 4 / v("per_gpu_tp4_mixed_GB") - 1) > 0.04, name
    for name, mb in {"fp8 with one byte scale per 16": n + n // 16,
                     "fp8 with no block scales": n}.items():
        _, allmx = _ckpt_gb(expert_bytes["nvfp4"], mb)
        # a missing scale array is too small to see at the page's precision;
        # a per-16 scale is not
        if "per 16" in name:
            assert abs(allmx / v("ckpt_mxfp8_GB") - 1) > 0.02, name
