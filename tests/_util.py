"""Shared helpers of the GPU parity tests: seeded inputs (synth), the oracle's
expected values, upload to the device, and the output tolerance."""
from __future__ import annotations

import numpy as np

import synth
from oracle import layer as L

OUT_RTOL = 2e-2   # max |gpu - oracle| / max |oracle| on the bf16 layer output


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_err(got_bits, ref_bits) -> float:
    g, r = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def oracle_cfg(w: synth.Workload, **kw) -> L.OracleConfig:
    return L.OracleConfig(hidden=w.hidden, ffn=w.ffn, num_experts=w.experts, top_k=w.top_k, fmt=w.fmt,
                          expert_begin=w.expert_begin, num_local=w.num_local, cap=w.cap, **kw)


def lib_cfg(bse, w: synth.Workload, max_tokens=None, **kw):
    return bse.Config(hidden=w.hidden, ffn=w.ffn, num_experts=w.experts, top_k=w.top_k, fmt=w.fmt,
                      expert_begin=w.expert_begin, num_local_experts=w.num_local, cap=w.cap,
                      max_tokens=max_tokens or w.tokens, **kw)


def expert_weights(w: synth.Workload, e: int, gain: float = 1.0, sigma: float = 0.02) -> dict:
    """Canonical-layout weights of expert e for workload w.  Gaussian
    workloads are encoded by the oracle's quantizer; the others are drawn as
    codes directly (synth.expert_direct_codes)."""
    if w.weights == "gaussian":
        g, u, d = synth.expert_float_weights(w.seed, e, w.hidden, w.ffn, sigma=sigma * gain)
        return L.quantize_expert_weights(w.fmt, g, u, d)
    return synth.expert_direct_codes(w.seed, e, w.hidden, w.ffn, w.fmt, gain=gain)


class ExpertSource:
    """Picklable weight source for the oracle: e -> canonical weights of
    expert e of workload w (what expert_weights returns), so the oracle's
    worker processes draw their own experts."""

    def __init__(self, w: synth.Workload, gain: float = 1.0, edge: bool = False):
        self.w, self.gain, self.edge = w, gain, edge

    def __call__(self, e: int) -> dict:
        if self.edge:
            return synth.expert_direct_codes(self.w.seed, e, self.w.hidden, self.w.ffn, self.w.fmt, gain=self.gain,
                                             edge=True)
        return expert_weights(self.w, e, self.gain)


ORACLE_WORKERS = 8


def stack_local(w: synth.Workload, gain: float = 1.0) -> dict:
    n = w.experts if w.num_local is None else w.num_local
    ews = [expert_weights(w, w.expert_begin + i, gain) for i in range(n)]
    keys = ("w13", "w13_sc", "w2", "w2_sc") + (("gs",) if w.fmt == "nvfp4" else ())
    return {k: np.stack([np.asarray(e[k]) for e in ews]) for k in keys}, ews


def to_dev(a: np.ndarray, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def inputs(w: synth.Workload, T: int | None = None):
    T = w.tokens if T is None else T
    x = synth.tokens(w.seed, T, w.hidden)
    wr = synth.router_weight(w.seed, w.experts, w.hidden)
    b = synth.router_bias(w.seed, w.experts, w.bias)
    return x, wr, b
