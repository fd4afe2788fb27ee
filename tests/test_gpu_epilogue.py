"""The expert epilogue's capped SwiGLU on the device (moe_cap_swiglu, the
same device function the gate/up GEMM epilogues call) against the oracle's
float64 evaluation, element by element.

The device takes tanh and the sigmoid from the hardware exponential and
reciprocal; tanh uses an odd series for |x| < 1/8, where 1 - 2/(e^{2|x|}+1)
would cancel.  Bound: relative error <= 2e-5 wherever |exact| >= 1e-30 (the
exponential's argument is rounded to fp32 first, about 5e-6 relative at
|x| = 80); below that, absolute error <= 1e-30 (for a gate below -88.7 the
fp32 e^{-g} overflows and the sigmoid is 0, where the exact SwiGLU value is
under 1e-36).
"""
import numpy as np
import pytest

from oracle import layer as L

pytestmark = pytest.mark.gpu

REL = 2e-5


def _inputs(seed=0, n=200000):
    g = np.random.default_rng(seed)
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
    small = sign * np.exp(g.uniform(np.log(1e-7), np.log(0.5), n))        # where tanh cancels
    mid = g.standard_normal(n) * 4.0
    big = sign * g.uniform(7.0, 90.0, n)
    a = np.concatenate([small, mid, big]).astype(np.float32)
    b = np.concatenate([g.permutation(small), g.permutation(mid), g.standard_normal(n) * 30]).astype(np.float32)
    return a, b


@pytest.mark.parametrize("form", [0, 1, 2, 3])
def test_cap_swiglu_relative_error(gpu_lib, form):
    import torch
    a, b = _inputs(form)
    cfg = gpu_lib.Config(hidden=256, ffn=128, num_experts=4, top_k=1, fmt="mxfp8", cap_form=form, cap=7.0)
    ga, gb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    h = torch.empty_like(ga)
    gpu_lib.cap_swiglu(cfg, ga, gb, h)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64)
    ocfg = L.OracleConfig(hidden=256, ffn=128, num_experts=4, top_k=1, fmt="mxfp8", cap_form=form, cap=7.0)
    ref = L.cap_swiglu(ocfg, a, b).astype(np.float64)
    normal = np.abs(ref) >= 1e-30
    rel = np.abs(got - ref)[normal] / np.abs(ref)[normal]
    assert rel.max() <= REL, (form, float(rel.max()))
    assert np.abs(got - ref)[~normal].max(initial=0.0) <= 1e-30
    # small arguments are where 1 - 2/(e^{2|x|}+1) loses its digits
    s = normal.copy()
    s[len(a) // 3:] = False
    assert (np.abs(got - ref)[s] / np.abs(ref)[s]).max() <= REL
