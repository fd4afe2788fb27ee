"""moe_forward_noalloc through the C ABI on the GPU: the same output as
moe_forward (bit-identical: the same kernels on the library's per-device
scratch buffer instead of a caller workspace), on two calls in a row, the
second with a smaller batch; and batches beyond the buffer rejected before
anything runs."""
import numpy as np
import pytest

import synth

from _util import inputs, lib_cfg, stack_local, to_dev

pytestmark = pytest.mark.gpu


def _setup(bse, w, max_tokens):
    cfg = lib_cfg(bse, w, max_tokens=max_tokens)
    stacked, _ = stack_local(w)
    wd = bse.prepare_weights(cfg, {k: to_dev(v) for k, v in stacked.items()})
    return cfg, bse.weights_struct(cfg, wd), wd


@pytest.mark.parametrize("key,t1,t2", [("decode_nvfp4", 64, 20), ("mid_mxfp8", 77, 5), ("many_rows", 700, 300)])
def test_noalloc_matches_forward_two_calls(gpu_lib, key, t1, t2):
    import torch
    from test_gpu_forward import SMALL
    bse = gpu_lib
    w = SMALL.get(key) or synth.WORKLOADS[key]
    cfg, cw, _keep = _setup(bse, w, t1)
    x, wr, b = inputs(w, t1)
    xt = to_dev(x.view(np.int16), torch.bfloat16)
    ws = bse.workspace(cfg)
    wrt, bt = to_dev(wr.view(np.int16), torch.bfloat16), to_dev(b)
    for T in (t1, t2):           # the second call is smaller: the buffer keeps the first one's contents
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
        bse.route(cfg, xt[:T], wrt, bt, ids, tw, None, ws)
        ref = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
        out = torch.full_like(ref, float("nan"))
        bse.forward(cfg, xt[:T], ids, tw, cw, ref, ws)
        bse.forward_noalloc(cfg, xt[:T], ids, tw, cw, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (key, T)


def test_noalloc_rejects_batches_beyond_the_buffer(gpu_lib):
    import torch
    bse = gpu_lib
    assert bse.noalloc_scratch_bytes() == 64 << 20
    w = synth.WORKLOADS["decode_nvfp4"]
    T = 270                      # the NVFP4 Inkling workspace for 270 tokens exceeds 64 MiB
    cfg = lib_cfg(bse, w, max_tokens=T)
    assert bse.workspace_size(bse.Config(fmt="nvfp4", max_tokens=T)) > 64 << 20
    x = torch.zeros((T, w.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, w.top_k), dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, w.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    fake = bse.CWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1)
    with pytest.raises(bse.MoeError) as e:
        bse.forward_noalloc(cfg, x, ids, tw, fake, out)
    assert e.value.status == -8
