"""The routed-expert MoE layer, written out as its plain definition (oracle
side, test infrastructure only).

What the layer computes (pages: TokenSpeed blog "What's new" table, MoE
row; Miles docs section 1, "Sigmoid-routed MoE" bullet; SGLang blog
"Performance", kernel-fusion bullet; SGLang cookbook section 2 "MegaMoE"):

1. Router logits z = x W_r^T (router weight in BF16: "the rest BF16", p3
   table, Checkpoint row).
2. Sigmoid scores s = sigmoid(z); the selection uses s + b (additive
   per-expert bias); top-k of 384 (k = 8).
3. Gate weights from the unbiased scores of the chosen experts.
4. Activations quantized per the layer's format (W4A4 for NVFP4 layers,
   W8A8 for MXFP8 layers; Miles docs section 5.3).
5. Per chosen expert: gate/up projection, capped SwiGLU, requantize, down
   projection.
6. Weighted combine of the k expert outputs per token.

Readings taken where the pages are silent (numbered R1, R2, ... throughout this package):

* R6  bias enters the selection only; gate weights use the plain sigmoid.
* R7  norm_topk (default on): gate weights are divided by their sum over the
      k chosen experts, then multiplied by routed_scale (default 1.0).
* R8  ties in the selection score go to the lower expert index; the chosen
      ids are listed in descending score order.  A token is a "near tie"
      when the k-th and (k+1)-th selection scores differ by less than 1e-6.
* R9  cap forms: SOFT_GATE_UP (default, "soft-capped" on p4) applies
      c*tanh(./c) to gate and up; HARD_GATE_UP clamps gate above at c and up
      to [-c, c]; SOFT_OUT caps the SwiGLU product; NONE is plain SwiGLU.
      SwiGLU is silu(g) * u.
* R10 rounding points: bf16 x in; fp32 logits and scores; quantized x; fp32
      gate, up and SwiGLU output h; quantized h (per (token, expert) row);
      fp32 expert output y; bf16 out.  Matmuls accumulate in float64 and
      round once to fp32.
* R11 x is quantized once per token, before dispatch.
* R12 expert-parallel share: only experts in [expert_begin,
      expert_begin + num_local) are computed; gate weights keep their
      normalisation over all k; out is the partial sum over local experts.
* R1  NVFP4 activation fp32 scale (act_gs): "row" (default) -- one scale per
      row over its full width, x rows for gate/up and (token, expert) h rows
      for down; "tensor" -- one scale over the whole activation tensor of the
      call (all T x rows; all local (token, expert) h rows); "static" -- the
      fixed scales act_gs_static = (x scale, h scale).  MXFP8 has no fp32
      scale and ignores act_gs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F

CAP_SOFT_GATE_UP = 0
CAP_HARD_GATE_UP = 1
CAP_SOFT_OUT = 2
CAP_NONE = 3

NEAR_TIE_GAP = 1e-6


@dataclass
class OracleConfig:
    hidden: int
    ffn: int
    num_experts: int
    top_k: int
    fmt: str                      # "nvfp4" | "mxfp8"
    expert_begin: int = 0
    num_local: int | None = None  # None -> all experts
    cap_form: int = CAP_SOFT_GATE_UP
    cap: float = 7.0
    norm_topk: bool = True
    routed_scale: float = 1.0
    act_gs: str = "row"                       # "row" | "tensor" | "static" (NVFP4 only)
    act_gs_static: tuple = (1.0, 1.0)         # (x scale, h scale) when act_gs == "static"

    @property
    def local(self) -> range:
        n = self.num_experts if self.num_local is None else self.num_local
        return range(self.expert_begin, self.expert_begin + n)


# --------------------------------------------------------------------------
# Router (steps 1-3)
# --------------------------------------------------------------------------

def _sigmoid64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def route(cfg: OracleConfig, x_bf16: np.ndarray, w_router_bf16: np.ndarray, bias: np.ndarray):
    """Sigmoid router with additive selection bias and top-k.

    x_bf16: uint16 [T, H]; w_router_bf16: uint16 [E, H]; bias: fp32 [E].
    Returns dict with logits fp32 [T,E], scores fp32 [T,E], sel fp32 [T,E],
    topk_ids int32 [T,k], topk_w fp32 [T,k], near_tie bool [T], gap fp64 [T].
    """
    x = F.bf16_bits_to_f32(x_bf16).astype(np.float64)
    w = F.bf16_bits_to_f32(w_router_bf16).astype(np.float64)
    z = (x @ w.T).astype(np.float32)                             # fp64 acc -> fp32
    s = _sigmoid64(z).astype(np.float32)
    sel = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    T, E = sel.shape
    k = cfg.top_k
    # descending score, ties to the lower index: sort keys (-sel, index)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -sel.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    sk = np.take_along_axis(sel, order[:, k - 1:k], axis=1)[:, 0].astype(np.float64)
    if k < E:
        sk1 = np.take_along_axis(sel, order[:, k:k + 1], axis=1)[:, 0].astype(np.float64)
        gap = sk - sk1
    else:
        gap = np.full(T, np.inf)
    near = gap < NEAR_TIE_GAP
    tw = gate_weights(cfg, s, ids)
    return dict(logits=z, scores=s, sel=sel, topk_ids=ids, topk_w=tw, near_tie=near, gap=gap)


def gate_weights(cfg: OracleConfig, scores: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Gate weights of the chosen experts from the unbiased sigmoid scores."""
    g = np.take_along_axis(scores, ids.astype(np.int64), axis=1).astype(np.float64)
    if cfg.norm_topk:
        tot = np.zeros(g.shape[0])
        for j in range(g.shape[1]):          # summed in j order
            tot = tot + g[:, j]
        g = g / tot[:, None]
    return (g * cfg.routed_scale).astype(np.float32)


# --------------------------------------------------------------------------
# Dispatch: stable sort of pair ids t*k+j by expert id (local experts only)
# --------------------------------------------------------------------------

def dispatch(cfg: OracleConfig, topk_ids: np.ndarray):
    """Returns expert_offsets int32 [n_local+1], sorted_pairs int32 [P_local]
    (pair ids ordered by (expert, pair id)), pair_pos int32 [T*k] (position
    of each pair in sorted_pairs, -1 for pairs whose expert is not local)."""
    ids = np.asarray(topk_ids, dtype=np.int64).ravel()
    loc = cfg.local
    is_local = (ids >= loc.start) & (ids < loc.stop)
    pair = np.nonzero(is_local)[0]
    order = np.argsort(ids[pair], kind="stable")
    sorted_pairs = pair[order].astype(np.int32)
    counts = np.bincount(ids[pair] - loc.start, minlength=len(loc))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pos = np.full(ids.shape[0], -1, dtype=np.int32)
    pos[sorted_pairs] = np.arange(sorted_pairs.shape[0], dtype=np.int32)
    return offsets, sorted_pairs, pos


# --------------------------------------------------------------------------
# Quantization of activations (step 4) and of weights
# --------------------------------------------------------------------------

def quantize_rows(fmt: str, v: np.ndarray, gs=None):
    """Activation quantization of fp32 rows; returns a dict.  NVFP4: with
    gs None each row takes its own fp32 scale (reading R1); otherwise every
    row takes the given fp32 scale (the per-tensor and static alternatives)."""
    if fmt == "mxfp8":
        c, s = F.quantize_mxfp8(v)
        return dict(codes=c, scales=s)
    if fmt == "nvfp4":
        if gs is None:
            c, s, g = F.quantize_nvfp4(v, domain="row")
        else:
            c, s, g = F.quantize_nvfp4(v, domain="static", gs=gs)
        return dict(codes=c, scales=s, gs=g)
    raise ValueError(fmt)


def act_scale(cfg: OracleConfig, site: int, v_all: np.ndarray):
    """The fp32 scale every row of an activation tensor shares under act_gs
    "tensor" (from the maximum over v_all, the whole tensor of the call) or
    "static" (act_gs_static[site]; site 0 = x, 1 = h); None for "row" and for
    MXFP8."""
    if cfg.fmt != "nvfp4" or cfg.act_gs == "row":
        return None
    if cfg.act_gs == "static":
        return np.float32(cfg.act_gs_static[site])
    if cfg.act_gs == "tensor":
        v_all = np.asarray(v_all, dtype=np.float32)
        A = np.max(np.abs(v_all)) if v_all.size else np.float32(0.0)
        return F.nvfp4_global_scale(A)[()]
    raise ValueError(cfg.act_gs)


def dequantize_rows(fmt: str, q: dict) -> np.ndarray:
    if fmt == "mxfp8":
        return F.dequantize_mxfp8(q["codes"], q["scales"])
    return F.dequantize_nvfp4(q["codes"], q["scales"], q["gs"])


def quantize_expert_weights(fmt: str, gate: np.ndarray, up: np.ndarray, down: np.ndarray):
    """Encode one expert's fp32 weights in the canonical layout.

    gate, up: [F, H]; down: [H, F] (rows = output features, columns = input).
    w13 rows are gate rows 0..F-1 then up rows F..2F-1 (reading R5).
    NVFP4: one fp32 scale per matrix (gate, up, down separately, R2).
    """
    if fmt == "mxfp8":
        c13, s13 = F.quantize_mxfp8(np.concatenate([gate, up], axis=0))
        c2, s2 = F.quantize_mxfp8(down)
        return dict(w13=c13, w13_sc=s13, w2=c2, w2_sc=s2)
    cg, sg, gg = F.quantize_nvfp4(gate, domain="tensor")
    cu, su, gu = F.quantize_nvfp4(up, domain="tensor")
    cd, sd, gd = F.quantize_nvfp4(down, domain="tensor")
    return dict(w13=np.concatenate([cg, cu], axis=0), w13_sc=np.concatenate([sg, su], axis=0),
                w2=cd, w2_sc=sd, gs=np.array([gg, gu, gd], dtype=np.float32))


def dequantize_expert(fmt: str, ew: dict):
    """Expert weights -> float64 (gate [F,H], up [F,H], down [H,F])."""
    if fmt == "mxfp8":
        w13 = F.dequantize_mxfp8(ew["w13"], ew["w13_sc"])
        w2 = F.dequantize_mxfp8(ew["w2"], ew["w2_sc"])
        Fd = w13.shape[0] // 2
        return w13[:Fd], w13[Fd:], w2
    Fd = ew["w13"].shape[0] // 2
    gs = np.asarray(ew["gs"], dtype=np.float32)
    g = F.dequantize_nvfp4(ew["w13"][:Fd], ew["w13_sc"][:Fd], gs[0])
    u = F.dequantize_nvfp4(ew["w13"][Fd:], ew["w13_sc"][Fd:], gs[1])
    d = F.dequantize_nvfp4(ew["w2"], ew["w2_sc"], gs[2])
    return g, u, d


# --------------------------------------------------------------------------
# Expert FFN (step 5)
# --------------------------------------------------------------------------

def cap_swiglu(cfg: OracleConfig, g32: np.ndarray, u32: np.ndarray) -> np.ndarray:
    """Capped SwiGLU of fp32 gate/up rows, evaluated in float64, rounded to fp32."""
    g = np.asarray(g32, dtype=np.float64)
    u = np.asarray(u32, dtype=np.float64)
    c = float(cfg.cap)
    if cfg.cap_form == CAP_SOFT_GATE_UP:
        g = c * np.tanh(g / c)
        u = c * np.tanh(u / c)
    elif cfg.cap_form == CAP_HARD_GATE_UP:
        g = np.minimum(g, c)
        u = np.clip(u, -c, c)
    h = g * _sigmoid64(g) * u
    if cfg.cap_form == CAP_SOFT_OUT:
        h = c * np.tanh(h / c)
    return h.astype(np.float32)


def expert_gate_up(cfg: OracleConfig, xq64: np.ndarray, wdeq) -> np.ndarray:
    """Gate/up projection and capped SwiGLU of one expert on rows of
    dequantized activations (float64 [n, H]); fp32 h [n, F]."""
    gate, up, _ = wdeq
    g = (xq64 @ gate.T).astype(np.float32)
    u = (xq64 @ up.T).astype(np.float32)
    return cap_swiglu(cfg, g, u)


def expert_down(cfg: OracleConfig, h: np.ndarray, wdeq, h_gs=None) -> np.ndarray:
    """h quantized per row (or with the shared scale h_gs, see act_scale),
    then the down projection; fp32 y [n, H]."""
    hq = dequantize_rows(cfg.fmt, quantize_rows(cfg.fmt, h, gs=h_gs))
    return (hq @ wdeq[2].T).astype(np.float32)


def expert_forward(cfg: OracleConfig, xq64: np.ndarray, wdeq, h_gs=None):
    """One expert on rows of dequantized activations (float64 [n, H]).
    Returns fp32 y [n, H] and the intermediate fp32 h [n, F]."""
    h = expert_gate_up(cfg, xq64, wdeq)
    return expert_down(cfg, h, wdeq, h_gs), h


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def moe_layer(cfg: OracleConfig, x_bf16, w_router_bf16, bias, expert_weights,
              tokens=None, topk_ids=None, topk_w=None, workers: int = 1):
    """Plain definition of the layer.

    expert_weights: callable e -> dict (canonical layout of expert e), or a
    dict/list indexable by local expert index (e - expert_begin).
    tokens: optional array of token indices; only those outputs are computed
    (the router still runs on those tokens only).
    topk_ids/topk_w: optional routing replay (replaces the router's choice).
    workers: experts are independent, so with workers > 1 they are evaluated
    by a pool of forked worker processes (the same arithmetic per expert;
    results are placed by expert).
    Under act_gs "tensor" the x scale is taken over all T tokens even when
    `tokens` selects some; the h scale needs every local pair's h, so
    `tokens` must then be None.
    Returns dict(out=bf16 bits uint16 [n, H], route=..., y=..., tokens=...).
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    T = x_bf16.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    per_tensor = cfg.fmt == "nvfp4" and cfg.act_gs == "tensor"
    if per_tensor and tokens is not None:
        raise ValueError("act_gs 'tensor': the h scale spans every token; pass tokens=None")
    xs = x_bf16[tok]
    r = route(cfg, xs, w_router_bf16, bias)
    ids = r["topk_ids"] if topk_ids is None else np.asarray(topk_ids, dtype=np.int32)[tok]
    tw = r["topk_w"] if topk_w is None else np.asarray(topk_w, dtype=np.float32)[tok]

    x_gs = act_scale(cfg, 0, F.bf16_bits_to_f32(x_bf16))
    xq = dequantize_rows(cfg.fmt, quantize_rows(cfg.fmt, F.bf16_bits_to_f32(xs), gs=x_gs))
    n, k = ids.shape
    H = cfg.hidden
    y = np.zeros((n, k, H), dtype=np.float32)
    have = np.zeros((n, k), dtype=bool)
    get = expert_weights if callable(expert_weights) else (lambda e: expert_weights[e - cfg.expert_begin])
    if not per_tensor:
        h_gs = act_scale(cfg, 1, None) if cfg.act_gs == "static" else None

        jobs = []
        for e in cfg.local:                               # expert-index order
            rows, slots = np.nonzero(ids == e)
            if rows.size:
                jobs.append((rows, slots, (cfg, xq[rows], get, e, h_gs)))
        if workers > 1 and len(jobs) > 1:
            ys = _run_pool(workers, get, [j[2] for j in jobs])
        else:
            ys = [_expert_job(j[2]) for j in jobs]
        for (rows, slots, _), ye in zip(jobs, ys):
            y[rows, slots] = ye
            have[rows, slots] = True
    else:
        # every local pair's h first: its shared scale spans all of them
        hs = {}
        for e in cfg.local:
            rows, slots = np.nonzero(ids == e)
            if rows.size:
                hs[e] = (rows, slots, expert_gate_up(cfg, xq[rows], dequantize_expert(cfg.fmt, get(e))))
        h_all = np.concatenate([v[2] for v in hs.values()]) if hs else np.zeros((0, cfg.ffn), np.float32)
        h_gs = act_scale(cfg, 1, h_all)
        for e, (rows, slots, h) in hs.items():
            y[rows, slots] = expert_down(cfg, h, dequantize_expert(cfg.fmt, get(e)), h_gs)
            have[rows, slots] = True

    out = combine(tw, y, have)
    return dict(out=out, route=r, topk_ids=ids, topk_w=tw, y=y, have=have, tokens=tok, x_gs=x_gs)


def _expert_job(job):
    """fp32 y of one expert's rows: job = (cfg, dequantized x rows, weight
    source, e, shared h scale or None); the weight source is get(e) when
    callable, else the expert's weights themselves."""
    cfg, xr, src, e, h_gs = job
    ew = src(e) if callable(src) else src
    ye, _ = expert_forward(cfg, xr, dequantize_expert(cfg.fmt, ew), h_gs)
    return ye


def _run_pool(workers: int, get, jobs):
    """_expert_job over jobs in forked worker processes.  A weight source
    that cannot be pickled is resolved here and its arrays are sent."""
    import multiprocessing
    import pickle
    from concurrent.futures import ProcessPoolExecutor
    try:
        pickle.dumps(get)
    except Exception:
        jobs = [(c, xr, get(e), e, g) for (c, xr, _, e, g) in jobs]
    with ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("fork")) as ex:
        return list(ex.map(_expert_job, jobs))


def combine(tw: np.ndarray, y: np.ndarray, have: np.ndarray) -> np.ndarray:
    """Weighted combine: out[t] = bf16_rne(sum_j tw[t, j] * y[t, j]) over the
    pairs that were computed (have), summed in float64 in fixed j order.
    tw fp32 [n, k]; y fp32 [n, k, H]; have bool [n, k].  Returns bf16 bits."""
    n, k = have.shape
    acc = np.zeros((n, y.shape[2]), dtype=np.float64)
    for j in range(k):                                    # fixed j order
        acc = acc + np.where(have[:, j:j + 1], tw[:, j:j + 1].astype(np.float64) * y[:, j].astype(np.float64), 0.0)
    return F.bf16_round_f64(acc)
