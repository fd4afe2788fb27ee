"""moe_route + moe_forward captured in a HIP graph and replayed.

The library allocates, frees, synchronizes and clears nothing on its own
(every buffer is the caller's, no memset is enqueued), so a whole layer step
can be captured once and replayed with new token data in the same buffers.
Each replay, separated by unrelated eager work and synchronizations, must
reproduce the eager result bit for bit (same kernels, same fixed orders).
Shapes cover the small-batch fused quantize + dispatch launch, the general
dispatch, both GEMM kernels (decode tiles and 128-row tiles) in both
formats, and the single-launch expert half.
"""
import numpy as np
import pytest

import synth

from _util import inputs, lib_cfg, stack_local, to_dev

pytestmark = pytest.mark.gpu

SHAPES = {
    "decode_tiles_nvfp4": synth.Workload("g1", "graph", 100, 1024, 32, 4, 512, "nvfp4", 31, weights="gaussian"),
    "big_tiles_mxfp8": synth.Workload("g2", "graph", 700, 256, 8, 2, 128, "mxfp8", 32, weights="gaussian"),
    "big_tiles_nvfp4_general_dispatch": synth.Workload("g3", "graph", 600, 256, 16, 8, 128, "nvfp4", 33,
                                                       weights="gaussian"),
    # the single-launch expert half (moe_forward_fused): its control words are cleared
    # by the quantize + dispatch kernel of the same step, not by a memset
    "single_launch_nvfp4": synth.Workload("g4", "graph", 100, 1024, 32, 4, 512, "nvfp4", 34, weights="gaussian"),
    "single_launch_mxfp8": synth.Workload("g5", "graph", 64, 512, 48, 8, 256, "mxfp8", 35, weights="gaussian"),
}
FUSED = {"single_launch_nvfp4", "single_launch_mxfp8"}


@pytest.mark.parametrize("key", list(SHAPES))
def test_graph_replays_match_eager(gpu_lib, key):
    import torch
    bse = gpu_lib
    w = SHAPES[key]
    T = w.tokens
    cfg = lib_cfg(bse, w, max_tokens=T)
    stacked, _ = stack_local(w)
    wd = bse.prepare_weights(cfg, {k: to_dev(v) for k, v in stacked.items()})
    x0, wr, b = inputs(w, T)
    wrt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(b).cuda()

    def tok(seed):
        xs = synth.tokens(seed, T, w.hidden)
        return torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).cuda()

    def buffers():
        ws = bse.workspace(cfg)
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
        out = torch.empty((T, w.hidden), dtype=torch.bfloat16, device="cuda")
        return ws, ids, tw, out

    def step(x, ws, ids, tw, out):
        bse.route(cfg, x, wrt, bt, ids, tw, None, ws)
        bse.forward(cfg, x, ids, tw, wd, out, ws, fused=key in FUSED)

    # eager references for three token batches (separate buffers)
    seeds = [w.seed, 1000 + w.seed, 2000 + w.seed]
    refs = []
    for sd in seeds:
        bufs = buffers()
        step(tok(sd), *bufs)
        torch.cuda.synchronize()
        refs.append((bufs[1].clone(), bufs[2].clone(), bufs[3].clone()))

    # capture one step on the graph's buffers (after an eager warm-up on them)
    xg = tok(seeds[0])
    gb = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(xg, *gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(xg, *gb)

    other = torch.randn(512, 512, device="cuda")
    for rep in range(2):
        for i, sd in enumerate(seeds):
            xg.copy_(tok(sd))
            gb[3].zero_()
            graph.replay()
            torch.cuda.synchronize()
            other = torch.tanh(other @ other.T / 512.0)   # unrelated eager work between replays
            torch.cuda.synchronize()
            ids_ref, tw_ref, out_ref = refs[i]
            assert torch.equal(gb[1], ids_ref), (rep, i)
            assert torch.equal(gb[2], tw_ref), (rep, i)
            assert torch.equal(gb[3].view(torch.int16), out_ref.view(torch.int16)), (rep, i)
