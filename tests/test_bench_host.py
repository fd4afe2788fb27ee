"""Host logic of bench.py, without a GPU: the per-expert byte model behind
the roofline's algorithmic bytes, the roofline and work arithmetic, and the
one-GPU contract of the command line."""
import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth
from oracle import layer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_expert_bytes_equal_the_oracle_encoding(fmt):
    """The byte model is the size of what the oracle's encoder produces for
    one expert (gate and up rows, then down rows, codes and block scales)."""
    w = synth.Workload("bb", "bytes", 4, 256, 8, 2, 128, fmt, 0, weights="gaussian")
    g, u, d = synth.expert_float_weights(0, 0, w.hidden, w.ffn)
    enc = L.quantize_expert_weights(fmt, g, u, d)
    b = bench.per_expert_bytes(w)
    for k in ("w13", "w13_sc", "w2", "w2_sc"):
        assert enc[k].nbytes == b[k], k
    assert b["gs"] == (np.asarray(enc["gs"], dtype=np.float32).nbytes if fmt == "nvfp4" else 0)


def test_inkling_expert_bytes():
    """Inkling 2 Small (hidden 4608, expert FFN 2304): the per-expert bytes the
    roofline's achieved GB/s are counted in."""
    nv = bench.per_expert_bytes(synth.WORKLOADS["decode_nvfp4"])
    assert nv["w13"] + nv["w13_sc"] == 11_943_936
    assert nv["w2"] + nv["w2_sc"] == 5_971_968
    assert sum(nv.values()) == 17_915_916
    mx = bench.per_expert_bytes(synth.WORKLOADS["decode_mxfp8"])
    assert mx["w13"] + mx["w13_sc"] == 21_897_216
    assert mx["w2"] + mx["w2_sc"] == 10_948_608
    assert sum(mx.values()) == 32_845_824


class _Cfg:
    def __init__(self, n):
        self.num_local = n


def test_work_counts_only_local_pairs_and_experts():
    torch = pytest.importorskip("torch")
    w = dataclasses.replace(synth.WORKLOADS["ep8_mxfp8"], tokens=3)   # experts 0..47 local of 384
    ids = np.array([[0, 1, 100, 200, 47, 48, 5, 6],
                    [0, 2, 101, 201, 300, 301, 302, 303],
                    [47, 383, 382, 381, 380, 379, 378, 377]], dtype=np.int32)
    st = {"w": w, "cfg": _Cfg(48), "per_expert": bench.per_expert_bytes(w), "ids": torch.from_numpy(ids)}
    wk = bench.work_of(st)
    assert wk["local_pairs"] == 8                 # 0 1 47 5 6 | 0 2 | 47
    assert wk["active"] == 6                      # {0, 1, 2, 5, 6, 47}
    pe = st["per_expert"]
    assert wk["expert_bytes"] == 6 * (pe["w13"] + pe["w13_sc"] + pe["w2"] + pe["w2_sc"])
    assert wk["flops_gu"] == 2.0 * 8 * 2 * w.ffn * w.hidden
    assert wk["flops"] == wk["flops_gu"] + 2.0 * 8 * w.ffn * w.hidden + 2.0 * 3 * w.experts * w.hidden


def test_roofline_hbm_and_mfma_arithmetic():
    w = synth.WORKLOADS["decode_nvfp4"]
    pe = bench.per_expert_bytes(w)
    wk = {"active": 121, "w13_bytes": pe["w13"] + pe["w13_sc"], "w2_bytes": pe["w2"] + pe["w2_sc"]}
    r = bench.roofline_of({"w": w, "per_expert": pe}, {"gate_up_ms": 0.2, "gate_up_ms_median": 0.25}, wk,
                          "canonical", False)
    assert (r["bound"], r["unit"], r["peak"]) == ("hbm", "GB/s", 8000.0)
    assert r["achieved"] == round(121 * 11_943_936 / 0.2e-3 / 1e9, 1)
    assert r["frac"] == round(r["achieved"] / 8000.0, 4)
    assert r["achieved_at_median"] == round(121 * 11_943_936 / 0.25e-3 / 1e9, 1)
    assert r["traffic"] is None                   # counters apply to the packed layout only

    w = synth.WORKLOADS["prefill_nvfp4"]
    pairs = 131072
    flops = 2.0 * pairs * 2 * w.ffn * w.hidden
    r = bench.roofline_of({"w": w, "per_expert": bench.per_expert_bytes(w)},
                          {"gate_up_ms": 5.0, "gate_up_ms_median": 4.0},
                          {"flops_gu": flops, "local_pairs": pairs}, "canonical", False)
    # NVFP4 runs the exact path on f16 MFMA: the f16 peak, with fp8 / fp4 fractions beside it
    assert (r["bound"], r["unit"], r["peak"], r["mfma_issued"]) == ("mfma", "TFLOP/s", 2500.0, "f16")
    assert r["achieved"] == round(flops / 5e-3 / 1e12, 1)
    assert r["frac_of_fp8_peak"] == round(flops / 5e-3 / 1e12 / 5000.0, 4)
    assert r["frac_of_fp4_peak"] == round(flops / 5e-3 / 1e12 / 10100.0, 4)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""
