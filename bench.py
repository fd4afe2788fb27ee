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

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-sub] [--flush]
    python bench.py --copy-calibration   # plain copy of known size (counter scale)

With the default workload the line also carries `sub_workloads`: the 16K
prefill chunk (the metric's other half, roofline against the MFMA peak), the
EP8 share and the MXFP8 decode batch, each measured the same way.
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


def expert_shapes(w, n: int) -> dict:
    """Byte shapes of n local experts' canonical arrays: gate and up rows then
    down rows, NVFP4 (two E2M1 codes per byte, one E4M3 scale per 16) or
    MXFP8 (one E4M3 code per byte, one E8M0 scale per 32)."""
    H, F = w.hidden, w.ffn
    nv = w.fmt == "nvfp4"
    return {"w13": (n, 2 * F, H // 2 if nv else H), "w13_sc": (n, 2 * F, H // (16 if nv else 32)),
            "w2": (n, H, F // 2 if nv else F), "w2_sc": (n, H, F // (16 if nv else 32))}


def per_expert_bytes(w) -> dict:
    """Bytes of one expert by array (the algorithmic bytes of the roofline),
    with the NVFP4 per-matrix fp32 scales (gate, up, down) under "gs"."""
    b = {k: int(np.prod(s[1:])) for k, s in expert_shapes(w, 1).items()}
    b["gs"] = 12 if w.fmt == "nvfp4" else 0
    return b


def upload_weights(w, bse_cfg):
    """Generate the local experts' direct-code weights and copy them to HBM."""
    import torch
    import synth
    n = bse_cfg.num_local
    H, F = w.hidden, w.ffn
    nv = w.fmt == "nvfp4"
    shapes = expert_shapes(w, n)
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
    return dev, per_expert_bytes(w)


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


# Weights of the touched experts for the oracle timing, drawn before the
# clock starts; module level so that the oracle's forked worker processes
# read them without copies.
_ORACLE_WEIGHTS = {}


class _CachedExperts:
    """Picklable weight source for the oracle: e -> the pre-drawn weights."""

    def __call__(self, e):
        return _ORACLE_WEIGHTS[e]


def host_cores() -> int:
    """CPU cores this process may use: its affinity set, capped by
    OMP_NUM_THREADS when that is set (the CPU share of a shared machine)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_baseline(w, x, wr, b, one_thread_tokens: int = 2):
    """The oracle (as it stands) timed on the host: the whole batch of the
    workload with every core (experts in one single-threaded worker process
    per core), and a 1-thread run on the first few tokens as one batch.  Timed: routing, x quantization, dequantization of the touched
    experts, float64 GEMMs, capped SwiGLU, h requantization, combine; the
    expert weights are drawn before the clock starts."""
    import threadpoolctl
    import synth
    from oracle import layer as L
    cfg = L.OracleConfig(hidden=w.hidden, ffn=w.ffn, num_experts=w.experts, top_k=w.top_k, fmt=w.fmt,
                         expert_begin=w.expert_begin, num_local=w.num_local, cap=w.cap)
    cores = host_cores()
    ids = L.route(cfg, x, wr, b)["topk_ids"]
    touched = sorted(set(int(e) for e in ids.ravel()) & set(cfg.local))
    _ORACLE_WEIGHTS.clear()
    for e in touched:
        _ORACLE_WEIGHTS[e] = synth.expert_direct_codes(w.seed, e, w.hidden, w.ffn, w.fmt) \
            if w.weights == "direct" else L.quantize_expert_weights(w.fmt, *synth.expert_float_weights(
                w.seed, e, w.hidden, w.ffn))
    src = _CachedExperts()
    # one BLAS thread per worker process (the workers inherit the limit)
    with threadpoolctl.threadpool_limits(limits=1):
        t0 = time.perf_counter()
        L.moe_layer(cfg, x, wr, b, src, workers=cores)
        t_all = time.perf_counter() - t0
    n1 = min(one_thread_tokens, x.shape[0])
    with threadpoolctl.threadpool_limits(limits=1):
        t0 = time.perf_counter()
        L.moe_layer(cfg, x[:n1], wr, b, src, workers=1)
        t_one = time.perf_counter() - t0
    _ORACLE_WEIGHTS.clear()
    T = x.shape[0]
    return {"value": round(T / t_all, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole batch: {T} tokens, {len(touched)} experts touched, {t_all:.1f} s on {cores} cores "
                      f"(experts in {cores} worker processes)",
            "one_thread": {"value": round(n1 / t_one, 4), "unit": "tokens/s", "cores": 1,
                           "sample": f"the first {n1} tokens as one batch, {t_one:.1f} s on 1 thread"}}


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


def make_state(w, layout: str):
    """Inputs, expert weights (in HBM), workspace and outputs of workload w."""
    import torch
    import block_scaled_expert_amd as bse
    import synth
    T, H, E, k = w.tokens, w.hidden, w.experts, w.top_k
    cfg = bse.Config(hidden=H, ffn=w.ffn, num_experts=E, top_k=k, fmt=w.fmt, expert_begin=w.expert_begin,
                     num_local_experts=w.num_local, cap=w.cap, max_tokens=T)
    x = synth.tokens(w.seed, T, H)
    wr = synth.router_weight(w.seed, E, H)
    b = synth.router_bias(w.seed, E, w.bias)
    t0 = time.time()
    wdev, per_expert = upload_weights(w, cfg)
    if layout == "packed":
        canon = wdev
        wdev = bse.prepare_weights(cfg, canon)
        torch.cuda.synchronize()
        del canon
    log(f"{w.key}: weights generated and uploaded in {time.time() - t0:.1f} s")
    st = dict(w=w, cfg=cfg, x=x, wr=wr, b=b, wdev=wdev, per_expert=per_expert, cw=bse.weights_struct(cfg, wdev))
    st["xt"] = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    st["wrt"] = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).cuda()
    st["bt"] = torch.from_numpy(b).cuda()
    st["ws"] = bse.workspace(cfg)
    st["ids"] = torch.empty((T, k), dtype=torch.int32, device="cuda")
    st["tw"] = torch.empty((T, k), dtype=torch.float32, device="cuda")
    st["out"] = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    return st


def measure(st, steps: int, warmup: int, fused: bool = False, graph: bool = False, flush: bool = False,
            route_forward: bool = False):
    """Warm-up, then the timed region of exactly `steps` steps (the gate/up
    kernel's HIP events recorded inside it), then `steps` more steps with an
    event pair around each (per-step median; with `flush`, a 1 GiB write
    between steps evicts the caches), then untimed steps with every stage's
    events."""
    import torch
    import block_scaled_expert_amd as bse
    cfg, cw = st["cfg"], st["cw"]
    xt, wrt, bt, ws, ids, tw, out = (st[n] for n in ("xt", "wrt", "bt", "ws", "ids", "tw", "out"))

    def step(events=None):
        if route_forward:
            bse.route_forward(cfg, xt, wrt, bt, ids, tw, None, cw, out, ws, events=events)
        else:
            bse.route(cfg, xt, wrt, bt, ids, tw, None, ws)
            bse.forward(cfg, xt, ids, tw, cw, out, ws, events=events, fused=fused)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = None
    if graph:
        # the whole step (route + forward) as one graph; no memsets are recorded
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step()
        torch.cuda.current_stream().wait_stream(s_cap)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()

    nst = len(bse.STAGES)
    gu = bse.STAGES.index("gate_up")

    def stage_events(all_stages):
        row = [torch.cuda.Event(enable_timing=True) if (all_stages or s // 2 == gu) else None
               for s in range(2 * nst)]
        for e in row:                # create the underlying HIP events
            if e is not None:
                e.record()
        return row

    # timed region: only the gate/up kernel's pair of events per step (each
    # recorded event adds about 2 us to the stream's timeline)
    evs = [stage_events(False) for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(steps):
        if g is not None:
            g.replay()
        else:
            step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / steps
    if g is not None:      # gate/up times from eager steps after the timed region
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
    gu_ms = [evs[i][2 * gu].elapsed_time(evs[i][2 * gu + 1]) for i in range(steps)]

    # per-step pass: an event pair around every step (median, spread)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, z in pairs:
        if flush_buf is not None:
            flush_buf.zero_()
        a.record()
        if g is not None:
            g.replay()
        else:
            step()
        z.record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(z) for a, z in pairs])
    del flush_buf

    n_stage = min(steps, 20)
    sevs = [stage_events(True) for _ in range(n_stage)]
    torch.cuda.synchronize()
    for i in range(n_stage):
        step(sevs[i])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([sevs[i][2 * s].elapsed_time(sevs[i][2 * s + 1]) for i in range(n_stage)]))
                for s, name in enumerate(bse.STAGES)}
    return dict(ms=ms, wall=wall, gate_up_ms=float(np.mean(gu_ms)), gate_up_ms_median=float(np.median(gu_ms)),
                step_ms_median=float(np.median(per_step)), step_ms_p10=float(np.percentile(per_step, 10)),
                step_ms_p90=float(np.percentile(per_step, 90)), stage_ms=stage_ms, n_stage=n_stage,
                flushed=flush)


def work_of(st):
    """Local pairs, active experts and the algorithmic bytes / flops of one step."""
    w, cfg, per_expert = st["w"], st["cfg"], st["per_expert"]
    T, H, E = w.tokens, w.hidden, w.experts
    ids_np = st["ids"].cpu().numpy()
    loc = range(w.expert_begin, w.expert_begin + cfg.num_local)
    local_pairs = int(np.isin(ids_np, list(loc)).sum())
    counts = np.bincount(ids_np.ravel(), minlength=E)
    active = int(len(set(ids_np.ravel().tolist()) & set(loc)))
    w13_bytes = per_expert["w13"] + per_expert["w13_sc"]
    w2_bytes = per_expert["w2"] + per_expert["w2_sc"]
    expert_bytes = active * (w13_bytes + w2_bytes + per_expert["gs"])
    flops_gu = 2.0 * local_pairs * 2 * w.ffn * H
    flops = flops_gu + 2.0 * local_pairs * w.ffn * H + 2.0 * T * E * H
    alg_bytes = expert_bytes + E * H * 2 + E * 4 + 2 * T * H * 2
    return dict(local_pairs=local_pairs, active=active, w13_bytes=w13_bytes, w2_bytes=w2_bytes,
                expert_bytes=expert_bytes, flops_gu=flops_gu, flops=flops, alg_bytes=alg_bytes,
                skew=float(counts.max() / counts.mean()), empty_experts=int((counts == 0).sum()))


def roofline_of(st, res, wk, layout: str, fused: bool):
    """Roofline of the dominant kernel (gate/up, or the single launch),
    timed by the HIP events recorded around it inside the timed region."""
    w = st["w"]
    T, H, E, k = w.tokens, w.hidden, w.experts, w.top_k
    decode = w.key.startswith("decode") or w.key == "tiny"
    gemm_kernel = ("k_expert_gemm" if gemm_source(w.key) == "gemm.hip"
                   else "k_expert_gemm_big_nv" if w.fmt == "nvfp4" else "k_expert_gemm_big_mx")
    t_mean, t_med = res["gate_up_ms"] * 1e-3, res["gate_up_ms_median"] * 1e-3
    pe = st["per_expert"]
    if fused and fused_applies(T, k, E):
        fb = wk["w13_bytes"] + wk["w2_bytes"] + pe["gs"]
        per = wk["active"] * fb
        tr = measured_traffic(w.key, "fused", fused=True) if layout == "packed" else None
        r = {"bound": "hbm", "achieved": round(per / t_mean / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "kernel": "k_moe_fused (gate/up, h quantization, down, combine)",
             "per_launch": f"{wk['active']} experts x {fb} B (w13 + w2 codes + scales)"}
        r["frac"] = round(r["achieved"] / HBM_PEAK_GBS, 4)
        r["achieved_at_median"] = round(per / t_med / 1e9, 1)
    elif decode or w.key.startswith("ep8"):
        per = wk["active"] * wk["w13_bytes"]
        tr = measured_traffic(w.key, "gate_up") if layout == "packed" else None
        r = {"bound": "hbm", "achieved": round(per / t_mean / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "kernel": gemm_kernel + " gate/up",
             "per_launch": f"{wk['active']} experts x {wk['w13_bytes']} B (w13 codes + scales)"}
        r["frac"] = round(r["achieved"] / HBM_PEAK_GBS, 4)
        r["achieved_at_median"] = round(per / t_med / 1e9, 1)
    else:
        issued = MFMA_ISSUED[w.fmt]
        per = wk["flops_gu"]
        tr = measured_traffic(w.key, "gate_up") if layout == "packed" else None
        ach = per / t_mean / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[issued], "unit": "TFLOP/s",
             "frac": round(ach / MFMA_PEAK_TFLOPS[issued], 4), "kernel": gemm_kernel + " gate/up",
             "mfma_issued": issued, "frac_of_fp8_peak": round(ach / MFMA_PEAK_TFLOPS["fp8"], 4),
             "frac_of_fp4_peak": round(ach / MFMA_PEAK_TFLOPS["fp4"], 4),
             "achieved_at_median": round(per / t_med / 1e12, 1),
             "per_launch": f"2 x {wk['local_pairs']} pairs x {2 * w.ffn} x {H} flop"}
        per = None
    r["traffic"] = tr
    if per is not None:
        r["traffic_over_algorithmic"] = None if tr is None else round(tr / per, 4)
    r["kernel_ms"] = round(res["gate_up_ms"], 4)
    r["kernel_ms_median"] = round(res["gate_up_ms_median"], 4)
    return r


def record_of(st, res, wk, layout, fused, graph):
    """Throughput, roofline and work of one measured workload."""
    w, cfg = st["w"], st["cfg"]
    ms = res["ms"]
    single = fused and fused_applies(w.tokens, w.top_k, w.experts)
    rec = {
        "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(res["step_ms_median"], 4),
        "ms_per_step_p10_p90": [round(res["step_ms_p10"], 4), round(res["step_ms_p90"], 4)],
        "dtype": {"nvfp4": "nvfp4 (W4A4, fp32 acc)", "mxfp8": "mxfp8 (W8A8, fp32 acc)"}[w.fmt],
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "experts": w.experts,
                   "top_k": w.top_k, "ffn": w.ffn, "format": w.fmt, "local_experts": cfg.num_local,
                   "weight_layout": layout,
                   "launch": ("hip_graph" if graph else "eager") + (", single-launch expert half" if single else "")},
        "roofline": roofline_of(st, res, wk, layout, fused),
        "tflops": round(wk["flops"] / (ms * 1e-3) / 1e12, 2),
        "expert_weight_GBs": round(wk["expert_bytes"] / (ms * 1e-3) / 1e9, 1),
        "expert_weight_frac_of_hbm": round(wk["expert_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "alg_GBs": round(wk["alg_bytes"] / (ms * 1e-3) / 1e9, 1),
        "active_experts": wk["active"], "local_pairs": wk["local_pairs"],
        "expert_load_max_over_mean": round(wk["skew"], 2), "empty_experts": wk["empty_experts"],
        "stage_ms": {k2: round(v, 4) for k2, v in res["stage_ms"].items()},
        "stage_ms_note": f"{res['n_stage']} untimed steps with every stage event recorded (each event adds ~2 us)",
        "wall_s_timed": round(res["wall"], 3),
    }
    if w.fmt == "nvfp4" and not (w.key.startswith("decode") or w.key.startswith("ep8") or w.key == "tiny"):
        rec["step_frac_of_f16_peak"] = round(wk["flops"] / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["f16"], 4)
    return rec


SUB_WORKLOADS = ("prefill_nvfp4", "ep8_mxfp8", "decode_mxfp8")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_nvfp4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the other workloads' records (16K prefill, EP8 share, MXFP8 decode)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (launch overhead removed)")
    ap.add_argument("--flush", action="store_true",
                    help="per-step pass: write a 1 GiB buffer between steps (caches evicted)")
    ap.add_argument("--layout", choices=["packed", "canonical"], default="packed",
                    help="expert weight layout (packed: moe_prepare_weights at load time)")
    ap.add_argument("--encode", choices=["nvfp4", "mxfp8"], default=None,
                    help="instead of the layer: time moe_encode_weights on bf16 experts of the Inkling shape")
    ap.add_argument("--encode-experts", type=int, default=64)
    ap.add_argument("--fused", action="store_true",
                    help="moe_forward_fused: the expert half as one launch")
    ap.add_argument("--route-forward", action="store_true",
                    help="moe_route_forward: routing, x quantization and dispatch in one launch (small batches)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="batch size other than the workload's (small-batch decode timings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the layer is measured on one GPU's "
              f"share (the EP8 workload is one expert-parallel rank's experts); no multi-GPU path is built.",
              file=sys.stderr)
        return 2

    import torch
    import synth

    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.encode:
        return encode_bench(args)

    # The other workloads of the metric (the 16K prefill chunk, the EP8 share,
    # the MXFP8 decode batch) are measured first, each with the same steps and
    # warm-up, then the main workload, whose line this is.  Every workload's
    # inputs and weights are put in HBM before any is measured, so the
    # measurements run back to back (drawing weights on the host between
    # them would leave the GPU idle, and its clocks low, just before a timed
    # region).
    sub_keys = [] if (args.no_sub or args.workload != "decode_nvfp4" or args.tokens) else list(SUB_WORKLOADS)
    w = synth.WORKLOADS[args.workload]
    if args.tokens:
        import dataclasses
        w = dataclasses.replace(w, tokens=args.tokens, name=f"{w.name} at {args.tokens} tokens")
    states = {}
    for key in sub_keys + [w.key]:
        wl = w if key == w.key else synth.WORKLOADS[key]
        log(f"workload {key}: {wl.name}")
        states[key] = make_state(wl, args.layout)
    subs = {}
    for key in sub_keys:
        st = states.pop(key)
        res = measure(st, args.steps, args.warmup, fused=args.fused, graph=args.graph, flush=args.flush)
        subs[key] = record_of(st, res, work_of(st), args.layout, args.fused, args.graph)
        del st

    st = states.pop(w.key)
    res = measure(st, args.steps, args.warmup, fused=args.fused, graph=args.graph, flush=args.flush,
                  route_forward=args.route_forward)
    wk = work_of(st)
    rec = record_of(st, res, wk, args.layout, args.fused, args.graph)
    if args.route_forward:
        rec["config"]["launch"] += ", moe_route_forward (routing + x quantization + dispatch in one launch)"
    line = {"metric": METRIC, "value": rec.pop("value"), "unit": rec.pop("unit"), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": rec.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": rec.pop("dtype"),
            "data": "synthetic (seeded; expert weights drawn as codes)"}
    cfgd = rec.pop("config")
    cfgd["parallelism"] = "single GPU"
    line["config"] = cfgd
    line.update(rec)
    if subs:
        line["sub_workloads"] = subs
        line["sub_workloads_note"] = ("the metric's other workloads, measured in this run before the main one with "
                                      "the same steps and warm-up")
    if not args.no_cpu:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w, st["x"], st["wr"], st["b"])
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
