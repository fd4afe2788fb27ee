"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = the whole hot path on one batch: moe_route (router GEMM,
sigmoid + bias + top-k) then moe_forward (activation quantization,
dispatch, gate/up GEMM + capped SwiGLU, h quantization, down GEMM,
combine), on seeded synthetic inputs already resident in HBM.

Default workload: the NVFP4 decode batch of 64 tokens (hidden 4608, 384
experts, top-8, expert FFN 2304).  Prints one JSON line with the throughput
(tokens/s), the roofline of the dominant kernel measured live with HIP
events on the stream the kernels run on, and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --copy-calibration   # plain copy of known size (counter scale)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s & HBM GB/s vs peak (decode b=64, 16K prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
MFMA_ISSUED = {"nvfp4": "f16", "mxfp8": "fp8"}   # MFMA type the expert GEMMs issue


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def upload_weights(w, bse_cfg):
    """Generate the local experts' direct-code weights and copy them to HBM."""
    import torch
    import synth
    n = bse_cfg.num_local
    H, F = w.hidden, w.ffn
    nv = w.fmt == "nvfp4"
    shapes = {"w13": (n, 2 * F, H // 2 if nv else H), "w13_sc": (n, 2 * F, H // (16 if nv else 32)),
              "w2": (n, H, F // 2 if nv else F), "w2_sc": (n, H, F // (16 if nv else 32))}
    dev = {k: torch.empty(s, dtype=torch.uint8, device="cuda") for k, s in shapes.items()}
    gs = np.zeros((n, 3), dtype=np.float32)
    for i in range(n):
        ew = synth.expert_direct_codes(w.seed, w.expert_begin + i, H, F, w.fmt)
        for k in shapes:
            dev[k][i].copy_(torch.from_numpy(ew[k]))
        if nv:
            gs[i] = ew["gs"]
    if nv:
        dev["gs"] = torch.from_numpy(gs).cuda()
    per_expert = {k: int(np.prod(s[1:])) for k, s in shapes.items()}
    per_expert["gs"] = 12 if nv else 0
    return dev, per_expert


def gemm_source(workload: str) -> str:
    """Source file of the expert GEMM kernel a workload runs: decode batches
    (a few rows per expert) take k_expert_gemm, prefill chunks and
    expert-parallel shares (128-row tiles) take k_expert_gemm_big_nv (NVFP4)
    or k_expert_gemm_big_mx (MXFP8)."""
    small = workload.startswith("decode") or workload == "tiny"
    return "gemm.hip" if small else "gemm_big.hip"


# headers each GEMM source includes (a change to any changes its kernels)
GEMM_HEADERS = {
    "gemm.hip": ("gemm_tile.h", "moe_common.h", "launch.h"),
    "gemm_big.hip": ("moe_common.h", "launch.h"),
    "fused.hip": ("gemm_tile.h", "quant_row.h", "combine.h", "moe_common.h", "launch.h"),
}


def gemm_source_sha256(fname: str) -> str:
    """sha256 over the GEMM source file and the headers it includes, in that
    order: a change to any of them changes the compiled kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in (fname, *GEMM_HEADERS[fname]):
        h.update(open(os.path.join(ROOT, "block_scaled_expert_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def fused_applies(T: int, k: int, E: int) -> bool:
    """moe_forward_fused runs its single expert-half launch for at most 4096 pairs
    and at most 48 expected rows per expert (work-list entries of <= 64 rows)."""
    return T * k <= 4096 and T * k <= 48 * E


def measured_traffic(workload: str, kernel: str, fused: bool = False):
    """HBM bytes (fetch + write) per launch of `kernel` ("gate_up" / "down",
    or "fused" for the single expert-half launch) recorded from rocprofv3 counters in
    profiles/traffic.json, if the kernel source and its headers have not
    changed since; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload + ("+fused" if fused else ""))
    fname = "fused.hip" if fused else gemm_source(workload)
    if (not rec or rec.get("source_file") != fname or rec.get("source_sha256") != gemm_source_sha256(fname)
            or kernel not in rec):
        return None
    return rec[kernel]["fetch_bytes"] + rec[kernel]["write_bytes"]


def cpu_baseline(w, x, wr, b, budget_s: float = 20.0):
    """The oracle (as it stands) on a bounded sample: whole layer outputs for a
    few tokens, routing included, using all host threads for BLAS."""
    import threadpoolctl
    import synth
    from oracle import layer as L
    cores = min(os.cpu_count() or 1, 16)
    cfg = L.OracleConfig(hidden=w.hidden, ffn=w.ffn, num_experts=w.experts, top_k=w.top_k, fmt=w.fmt,
                         expert_begin=w.expert_begin, num_local=w.num_local, cap=w.cap)
    cache = {}

    def ew(e):
        if e not in cache:
            cache[e] = synth.expert_direct_codes(w.seed, e, w.hidden, w.ffn, w.fmt)
        return cache[e]

    done, t_used = 0, 0.0
    with threadpoolctl.threadpool_limits(limits=cores):
        used = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
        while t_used < budget_s and done < x.shape[0]:
            tok = [done]
            for e in L.route(cfg, x[tok], wr, b)["topk_ids"][0]:   # draw the inputs outside the clock
                ew(int(e))
            t0 = time.perf_counter()
            L.moe_layer(cfg, x, wr, b, ew, tokens=tok)
            t_used += time.perf_counter() - t0
            done += 1
    return {"value": done / t_used, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{done} of {x.shape[0]} tokens of the same workload, one at a time (route, quantize, "
                      f"dequantize the token's experts, fp64 GEMMs, capped SwiGLU, requantize, combine); "
                      f"{t_used:.1f} s of CPU work"}


def encode_bench(args) -> int:
    """Time the GPU weight encoder on n bf16 experts of the Inkling shape
    (gate/up [n][2][2304][4608], down [n][4608][2304], values N(0, 0.02^2)).
    A step encodes all of them.  Algorithmic bytes per element: 2 read
    (bf16) plus the encoded bytes written (NVFP4 0.5625, MXFP8 1.03125)."""
    import torch
    import block_scaled_expert_amd as bse
    fmt, n, H, Fd = args.encode, args.encode_experts, 4608, 2304
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    wg = (torch.randn((2 * n, Fd, H), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wd = (torch.randn((n, H, Fd), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    nv = fmt == "nvfp4"
    c13 = torch.empty((2 * n, Fd, H // 2 if nv else H), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((2 * n, Fd, H // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    c2 = torch.empty((n, H, Fd // 2 if nv else Fd), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((n, H, Fd // (16 if nv else 32)), dtype=torch.uint8, device="cuda")
    gs = torch.empty((n, 3), dtype=torch.float32, device="cuda") if nv else None
    ws = torch.empty(2 * n, dtype=torch.int32, device="cuda") if nv else None

    def step():
        bse.encode_weights(fmt, wg, c13, s13, gs=gs, gs_group=2, gs_stride=3, ws=ws)
        bse.encode_weights(fmt, wd, c2, s2, gs=gs.view(-1)[2:] if nv else None, gs_group=1, gs_stride=3, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    elems = 3.0 * n * Fd * H
    alg = elems * (2 + (0.5 + 1 / 16 if nv else 1 + 1 / 32)) + (3 * n * 4 if nv else 0)
    gbs = alg / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "expert weight encode throughput (bf16 -> checkpoint format, scales recomputed)",
        "value": round(n / (ms * 1e-3), 1), "unit": "experts/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, " + fmt + " out", "data": "synthetic (N(0, 0.02^2) bf16)",
        "config": {"workload": f"encode {n} experts, H4608, F2304", "experts": n, "format": fmt},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "per_launch": f"{int(elems)} elements x (2 B read + encoded bytes written)"},
    }))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_nvfp4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (launch overhead removed)")
    ap.add_argument("--layout", choices=["packed", "canonical"], default="packed",
                    help="expert weight layout (packed: moe_prepare_weights at load time)")
    ap.add_argument("--encode", choices=["nvfp4", "mxfp8"], default=None,
                    help="instead of the layer: time moe_encode_weights on bf16 experts of the Inkling shape")
    ap.add_argument("--encode-experts", type=int, default=64)
    ap.add_argument("--fused", action="store_true",
                    help="moe_forward_fused: the expert half as one launch")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer is measured on one GPU's "
              f"share, see DESIGN.md for how it would shard.", file=sys.stderr)
        return 2

    import torch
    import block_scaled_expert_amd as bse
    import synth

    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.encode:
        return encode_bench(args)

    w = synth.WORKLOADS[args.workload]
    T, H, E, k = w.tokens, w.hidden, w.experts, w.top_k
    log(f"workload {w.key}: {w.name}")
    cfg = bse.Config(hidden=H, ffn=w.ffn, num_experts=E, top_k=k, fmt=w.fmt, expert_begin=w.expert_begin,
                     num_local_experts=w.num_local, cap=w.cap, max_tokens=T)
    x = synth.tokens(w.seed, T, H)
    wr = synth.router_weight(w.seed, E, H)
    b = synth.router_bias(w.seed, E, w.bias)
    t0 = time.time()
    wdev, per_expert = upload_weights(w, cfg)
    log(f"weights generated and uploaded in {time.time() - t0:.1f} s")
    if args.layout == "packed":
        canon = wdev
        wdev = bse.prepare_weights(cfg, canon)
        torch.cuda.synchronize()
        del canon
    cw = bse.weights_struct(cfg, wdev)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wrt = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(b).cuda()
    ws = bse.workspace(cfg)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step(events=None):
        bse.route(cfg, xt, wrt, bt, ids, tw, None, ws)
        bse.forward(cfg, xt, ids, tw, cw, out, ws, events=events, fused=args.fused)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # the whole step (route + forward) as one graph; no memsets are recorded
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step()
        torch.cuda.current_stream().wait_stream(s_cap)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()

    # Timed steps record only the gate/up kernel's pair of events (every
    # recorded event adds about 2 us to the stream's timeline); the full
    # per-stage breakdown comes from untimed steps afterwards.
    nst = len(bse.STAGES)
    gu = bse.STAGES.index("gate_up")

    def stage_events(all_stages):
        row = [torch.cuda.Event(enable_timing=True) if (all_stages or s // 2 == gu) else None
               for s in range(2 * nst)]
        for e in row:                # create the underlying HIP events
            if e is not None:
                e.record()
        return row

    evs = [stage_events(False) for _ in range(args.steps)]
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps
    if graph is not None:      # gate/up times from eager steps after the timed region
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
    gate_up_ms = float(np.mean([evs[i][2 * gu].elapsed_time(evs[i][2 * gu + 1]) for i in range(args.steps)]))
    n_stage = min(args.steps, 20)
    sevs = [stage_events(True) for _ in range(n_stage)]
    torch.cuda.synchronize()
    for i in range(n_stage):
        step(sevs[i])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([sevs[i][2 * s].elapsed_time(sevs[i][2 * s + 1]) for i in range(n_stage)]))
                for s, name in enumerate(bse.STAGES)}

    # work of one step
    ids_np = ids.cpu().numpy()
    loc = range(w.expert_begin, w.expert_begin + cfg.num_local)
    local_pairs = int(np.isin(ids_np, list(loc)).sum())
    active = int(len(set(ids_np.ravel().tolist()) & set(loc)))
    w13_bytes = per_expert["w13"] + per_expert["w13_sc"]
    w2_bytes = per_expert["w2"] + per_expert["w2_sc"]
    expert_bytes = active * (w13_bytes + w2_bytes + per_expert["gs"])
    flops_gu = 2.0 * local_pairs * 2 * w.ffn * H
    flops_dn = 2.0 * local_pairs * w.ffn * H
    flops = flops_gu + flops_dn + 2.0 * T * E * H
    alg_bytes = expert_bytes + E * H * 2 + E * 4 + 2 * T * H * 2

    decode = w.key.startswith("decode") or w.key == "tiny"
    gemm_kernel = ("k_expert_gemm" if gemm_source(w.key) == "gemm.hip"
                   else "k_expert_gemm_big_nv" if w.fmt == "nvfp4" else "k_expert_gemm_big_mx")
    single = args.fused and fused_applies(T, k, E)
    if single:
        # the single launch: both expert GEMMs. weights per launch
        fb = w13_bytes + w2_bytes + per_expert["gs"]
        achieved = active * fb / (gate_up_ms * 1e-3) / 1e9
        tr = measured_traffic(w.key, "fused", fused=True) if args.layout == "packed" else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr,
                "traffic_over_algorithmic": None if tr is None else round(tr / (active * fb), 4),
                "kernel": "k_moe_fused (gate/up, h quantization, down, combine)",
                "per_launch": f"{active} experts x {fb} B (w13 + w2 codes + scales)"}
    elif decode or w.key.startswith("ep8"):
        achieved = active * w13_bytes / (gate_up_ms * 1e-3) / 1e9
        tr = measured_traffic(w.key, "gate_up") if args.layout == "packed" else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr,
                "traffic_over_algorithmic": None if tr is None else round(tr / (active * w13_bytes), 4),
                "kernel": gemm_kernel + " gate/up", "per_launch": f"{active} experts x {w13_bytes} B (w13 codes + scales)"}
    else:
        issued = MFMA_ISSUED[w.fmt]
        achieved = flops_gu / (gate_up_ms * 1e-3) / 1e12
        tr = measured_traffic(w.key, "gate_up") if args.layout == "packed" else None
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS[issued], "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS[issued], 4), "traffic": tr,
                "kernel": gemm_kernel + " gate/up", "mfma_issued": issued,
                "frac_of_fp8_peak": round(achieved / MFMA_PEAK_TFLOPS["fp8"], 4),
                "frac_of_fp4_peak": round(achieved / MFMA_PEAK_TFLOPS["fp4"], 4),
                "per_launch": f"2 x {local_pairs} pairs x {2 * w.ffn} x {H} flop"}

    res = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"nvfp4": "nvfp4 (W4A4, fp32 acc)", "mxfp8": "mxfp8 (W8A8, fp32 acc)"}[w.fmt],
        "data": "synthetic (seeded; expert weights drawn as codes)",
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": E, "top_k": k, "ffn": w.ffn,
                   "format": w.fmt, "local_experts": cfg.num_local, "weight_layout": args.layout,
                   "launch": ("hip_graph" if args.graph else "eager") + (", single-launch expert half" if single
                                                                          else ""),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "expert_weight_GBs": round(expert_bytes / (ms * 1e-3) / 1e9, 1),
        "alg_GBs": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "active_experts": active, "local_pairs": local_pairs,
        "gate_up_ms": round(gate_up_ms, 4),
        "stage_ms": {k2: round(v, 4) for k2, v in stage_ms.items()},
        "stage_ms_note": f"{n_stage} untimed steps with every stage event recorded (each event adds ~2 us)",
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(w, x, wr, b, args.cpu_budget)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
