"""Python binding of libmoe.so, the gfx950 routed-expert MoE library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels on the caller's current torch stream.  The functions mirror the C
ABI in include/moe.h (moe_route, moe_dispatch, moe_quantize_act,
moe_forward, moe_forward_fused, moe_forward_fused_status, moe_route_forward,
moe_forward_noalloc, moe_cap_swiglu, moe_workspace_size,
moe_noalloc_scratch_bytes, moe_check_arch, moe_status_string, the weight
encoder and decoder).
Tensors must be contiguous and on the current CUDA (HIP) device; apart from
moe_forward_noalloc's fixed device array the library never allocates, so
callers pass outputs and a workspace.

There is no fallback: if the built library is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BSE_MOE_LIB") or os.path.join(HERE, "libmoe.so")

FMT_NVFP4, FMT_MXFP8 = 1, 2
FMTS = {"nvfp4": FMT_NVFP4, "mxfp8": FMT_MXFP8}
CAP_SOFT_GATE_UP, CAP_HARD_GATE_UP, CAP_SOFT_OUT, CAP_NONE = 0, 1, 2, 3
DTYPE_BF16, DTYPE_F32 = 0, 1
ACT_GS_PER_ROW, ACT_GS_PER_TENSOR, ACT_GS_STATIC = 0, 1, 2
ACT_GS_SCRATCH_BYTES = 1028   # moe_quantize_act's scratch for a per-tensor NVFP4 scale
STAGES = ("quant_x", "dispatch", "gate_up", "quant_h", "down", "combine")

EXPORTED = ("moe_status_string", "moe_check_arch", "moe_validate_config", "moe_workspace_size",
            "moe_quantize_act", "moe_route", "moe_dispatch", "moe_prepare_weights", "moe_forward",
            "moe_forward_fused", "moe_forward_fused_status", "moe_cap_swiglu", "moe_encode_weights",
            "moe_decode_weights", "moe_forward_noalloc", "moe_noalloc_scratch_bytes", "moe_route_forward")
LAYOUT_CANONICAL, LAYOUT_PACKED = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class CConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_begin", ctypes.c_int32),
                ("num_local_experts", ctypes.c_int32), ("fmt", ctypes.c_int32), ("cap_form", ctypes.c_int32),
                ("cap", ctypes.c_float), ("norm_topk", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("max_tokens", ctypes.c_int32), ("act_gs", ctypes.c_int32), ("act_gs_static", ctypes.c_float * 2)]


class CWeights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_sc", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_sc", ctypes.c_void_p), ("gs", ctypes.c_void_p), ("layout", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (built by block_scaled_expert_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_scaled_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_check_arch.argtypes = [ctypes.c_char_p]
    lib.moe_validate_config.argtypes = [ctypes.POINTER(CConfig)]
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(CConfig), ctypes.POINTER(sz)]
    lib.moe_quantize_act.argtypes = [ctypes.POINTER(CConfig), i32, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_cap_swiglu.argtypes = [ctypes.POINTER(CConfig), vp, vp, ctypes.c_int64, vp, vp]
    lib.moe_forward_fused_status.argtypes = [ctypes.POINTER(CConfig), i32, vp, sz, vp, vp]
    lib.moe_encode_weights.argtypes = [i32, i32, vp, i32, i32, i32, vp, vp, vp, i32, i32, vp, sz, vp]
    lib.moe_decode_weights.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.moe_route.argtypes = [ctypes.POINTER(CConfig), vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_dispatch.argtypes = [ctypes.POINTER(CConfig), vp, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_prepare_weights.argtypes = [ctypes.POINTER(CConfig), ctypes.POINTER(CWeights), ctypes.POINTER(CWeights),
                                        vp]
    lib.moe_forward.argtypes = [ctypes.POINTER(CConfig), vp, i32, vp, vp, ctypes.POINTER(CWeights), vp, vp,
                                sz, vp, vp]
    lib.moe_forward_fused.argtypes = lib.moe_forward.argtypes
    lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(CConfig), vp, i32, vp, vp, ctypes.POINTER(CWeights), vp, vp]
    lib.moe_noalloc_scratch_bytes.argtypes = []
    lib.moe_route_forward.argtypes = [ctypes.POINTER(CConfig), vp, i32, vp, vp, vp, vp, vp, ctypes.POINTER(CWeights),
                                      vp, vp, sz, vp, vp]
    for name in EXPORTED:
        if name != "moe_status_string":
            getattr(lib, name).restype = ctypes.c_int
    lib.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def check_arch(arch: str) -> int:
    return load().moe_check_arch(arch.encode())


@dataclass
class Config:
    hidden: int = 4608
    ffn: int = 2304
    num_experts: int = 384
    top_k: int = 8
    fmt: str = "nvfp4"
    expert_begin: int = 0
    num_local_experts: int | None = None
    cap_form: int = CAP_SOFT_GATE_UP
    cap: float = 7.0
    norm_topk: bool = True
    routed_scale: float = 1.0
    max_tokens: int = 64
    act_gs: int = ACT_GS_PER_ROW
    act_gs_static: tuple = (1.0, 1.0)

    @property
    def num_local(self) -> int:
        return self.num_experts if self.num_local_experts is None else self.num_local_experts

    def c(self) -> CConfig:
        if self.fmt not in FMTS:
            raise ValueError(f"unknown format {self.fmt!r}")
        return CConfig(self.hidden, self.ffn, self.num_experts, self.top_k, self.expert_begin, self.num_local,
                       FMTS[self.fmt], self.cap_form, self.cap, int(bool(self.norm_topk)), self.routed_scale,
                       self.max_tokens, self.act_gs, (ctypes.c_float * 2)(*self.act_gs_static))


def _ok(status: int, what: str) -> None:
    if status != 0:
        raise MoeError(status, what)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def workspace_size(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    cc = cfg.c()
    _ok(load().moe_workspace_size(ctypes.byref(cc), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def workspace(cfg: Config, device="cuda"):
    import torch
    return torch.empty(workspace_size(cfg), dtype=torch.uint8, device=device)


def quantize_act(cfg, x, codes, scales, row_gs=None, site: int = 0, ws=None) -> None:
    """NVFP4 / MXFP8 quantization of a bf16 or fp32 [rows, cols] tensor in
    cfg's format and activation-scale mode (cfg: a Config, or a format name
    for the per-row default).  site 0: gate/up input x, 1: down input h.
    ws: uint8 scratch of at least ACT_GS_SCRATCH_BYTES for NVFP4 per-tensor
    scales."""
    import torch
    if isinstance(cfg, str):
        cfg = Config(fmt=cfg)
    rows, cols = x.shape
    dt = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bfloat16 or float32")
    nv = cfg.fmt == "nvfp4"
    _ptr(x, name="x")
    cc = cfg.c()
    args = (ctypes.byref(cc), site, dt, _ptr(x), rows, cols,
            _ptr(codes, torch.uint8, (rows, cols // 2 if nv else cols), "codes"),
            _ptr(scales, torch.uint8, (rows, cols // (16 if nv else 32)), "scales"),
            _ptr(row_gs, torch.float32, (rows,), "row_gs") if nv else None,
            _ptr(ws, torch.uint8, None, "ws"), 0 if ws is None else ws.numel(), _stream())
    _ok(load().moe_quantize_act(*args), "moe_quantize_act")


def cap_swiglu(cfg: Config, g, u, h) -> None:
    """The expert epilogue's capped SwiGLU on fp32 tensors of equal size."""
    import torch
    n = g.numel()
    cc = cfg.c()
    _ok(load().moe_cap_swiglu(ctypes.byref(cc), _ptr(g, torch.float32, None, "g"),
                              _ptr(u, torch.float32, (n,) if u.dim() == 1 else None, "u"), n,
                              _ptr(h, torch.float32, None, "h"), _stream()), "moe_cap_swiglu")


def forward_fused_status(cfg: Config, T: int, ws, err) -> None:
    """err (int32 device tensor of one element) <- the error word of the last
    moe_forward_fused call on ws for T tokens (0: every wait was met)."""
    import torch
    cc = cfg.c()
    _ok(load().moe_forward_fused_status(ctypes.byref(cc), T, _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
                                        _ptr(err, torch.int32, (1,), "err"), _stream()),
        "moe_forward_fused_status")


def _check_gs(gs, nmat: int, group: int, stride: int) -> None:
    if gs is None or group < 1 or stride < group:
        raise ValueError("NVFP4 needs gs, gs_group >= 1 and gs_stride >= gs_group")
    need = ((nmat - 1) // group) * stride + (nmat - 1) % group + 1 if nmat > 0 else 0
    if gs.numel() < need:
        raise ValueError(f"gs must hold at least {need} floats")


def encode_weights(fmt: str, w, codes, scales, gs=None, gs_group: int = 1, gs_stride: int = 1,
                   ws=None) -> None:
    """Matrices w [nmat, rows, cols] (bf16 or fp32) to NVFP4 (one fp32 scale
    per matrix, recomputed from its max |w|, written to gs[(m // gs_group) *
    gs_stride + m % gs_group]; ws: int32 scratch of at least nmat elements)
    or MXFP8.  codes / scales: uint8 [nmat, rows, cols/2 or cols] and
    [nmat, rows, cols/16 or cols/32]."""
    import torch
    nmat, rows, cols = w.shape
    dt = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(w.dtype)
    if dt is None:
        raise ValueError("w must be bfloat16 or float32")
    nv = fmt == "nvfp4"
    _ptr(w, name="w")
    if nv:
        _check_gs(gs, nmat, gs_group, gs_stride)
        if ws is None or ws.numel() < nmat:
            raise ValueError(f"ws must hold at least {nmat} int32")
    args = (FMTS[fmt], dt, _ptr(w), nmat, rows, cols,
            _ptr(codes, torch.uint8, (nmat, rows, cols // 2 if nv else cols), "codes"),
            _ptr(scales, torch.uint8, (nmat, rows, cols // (16 if nv else 32)), "scales"),
            _ptr(gs, torch.float32, None, "gs") if nv else None, gs_group, gs_stride,
            _ptr(ws, torch.int32, None, "ws") if nv else None,
            (ws.numel() * 4) if (nv and ws is not None) else 0, _stream())
    _ok(load().moe_encode_weights(*args), "moe_encode_weights")


def decode_weights(fmt: str, codes, scales, out, gs=None, gs_group: int = 1, gs_stride: int = 1) -> None:
    """The fp32 values [nmat, rows, cols] of encoded matrices (see encode_weights)."""
    import torch
    nmat, rows, cols = out.shape
    nv = fmt == "nvfp4"
    if nv:
        _check_gs(gs, nmat, gs_group, gs_stride)
    args = (FMTS[fmt], _ptr(codes, torch.uint8, (nmat, rows, cols // 2 if nv else cols), "codes"),
            _ptr(scales, torch.uint8, (nmat, rows, cols // (16 if nv else 32)), "scales"),
            _ptr(gs, torch.float32, None, "gs") if nv else None, gs_group, gs_stride, nmat, rows, cols,
            _ptr(out, torch.float32, None, "out"), _stream())
    _ok(load().moe_decode_weights(*args), "moe_decode_weights")


def route(cfg: Config, x, w_router, bias, topk_ids, topk_w, near_tie, ws) -> None:
    import torch
    T = x.shape[0]
    H, E, k = cfg.hidden, cfg.num_experts, cfg.top_k
    cc = cfg.c()
    _ok(load().moe_route(ctypes.byref(cc), _ptr(x, torch.bfloat16, (T, H), "x"), T,
                         _ptr(w_router, torch.bfloat16, (E, H), "w_router"),
                         _ptr(bias, torch.float32, (E,), "bias"),
                         _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                         _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                         _ptr(near_tie, torch.uint8, (T,), "near_tie"),
                         _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()), "moe_route")


def dispatch(cfg: Config, topk_ids, expert_offsets, sorted_pairs=None, pair_pos=None, ws=None) -> None:
    import torch
    T = topk_ids.shape[0]
    P = T * cfg.top_k
    cc = cfg.c()
    _ok(load().moe_dispatch(ctypes.byref(cc), _ptr(topk_ids, torch.int32, (T, cfg.top_k), "topk_ids"), T,
                            _ptr(expert_offsets, torch.int32, (cfg.num_local + 1,), "expert_offsets"),
                            _ptr(sorted_pairs, torch.int32, None, "sorted_pairs"),
                            _ptr(pair_pos, torch.int32, (P,), "pair_pos"),
                            _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()), "moe_dispatch")


def weights_struct(cfg: Config, w: dict) -> CWeights:
    """w: dict of device tensors w13, w13_sc, w2, w2_sc (uint8), gs (fp32,
    NVFP4) and optionally layout (LAYOUT_CANONICAL by default)."""
    import torch
    H, F, n = cfg.hidden, cfg.ffn, cfg.num_local
    nv = cfg.fmt == "nvfp4"
    shapes = {
        "w13": (n, 2 * F, H // 2 if nv else H), "w13_sc": (n, 2 * F, H // (16 if nv else 32)),
        "w2": (n, H, F // 2 if nv else F), "w2_sc": (n, H, F // (16 if nv else 32)),
    }
    ptrs = {k: _ptr(w[k], torch.uint8, s, k) for k, s in shapes.items()}
    gs = _ptr(w["gs"], torch.float32, (n, 3), "gs") if nv else None
    return CWeights(ptrs["w13"], ptrs["w13_sc"], ptrs["w2"], ptrs["w2_sc"], gs, int(w.get("layout", LAYOUT_CANONICAL)))


def prepare_weights(cfg: Config, w: dict) -> dict:
    """Repack canonical expert weights into the packed layout (new device
    tensors of the same shapes; gs is shared)."""
    import torch
    src = weights_struct(cfg, w)
    out = {k: torch.empty_like(w[k]) for k in ("w13", "w13_sc", "w2", "w2_sc")}
    if "gs" in w:
        out["gs"] = w["gs"]
    out["layout"] = LAYOUT_PACKED
    dst = weights_struct(cfg, out)
    cc = cfg.c()
    _ok(load().moe_prepare_weights(ctypes.byref(cc), ctypes.byref(src), ctypes.byref(dst), _stream()),
        "moe_prepare_weights")
    return out


def forward(cfg: Config, x, topk_ids, topk_w, weights, out, ws, events=None, fused: bool = False) -> None:
    """weights: dict of device tensors or a CWeights built by weights_struct.
    events: optional list of 2*6 torch.cuda.Event (stage timing).
    fused: call moe_forward_fused (the expert half in one launch) instead of moe_forward."""
    import torch
    T = x.shape[0]
    H, k = cfg.hidden, cfg.top_k
    cw = weights if isinstance(weights, CWeights) else weights_struct(cfg, weights)
    ev = None
    if events is not None:
        if len(events) != 2 * len(STAGES):
            raise ValueError("events must hold 2 per stage")
        ev = (ctypes.c_void_p * len(events))(*[e.cuda_event if e is not None else None for e in events])
    cc = cfg.c()
    fn = load().moe_forward_fused if fused else load().moe_forward
    _ok(fn(ctypes.byref(cc), _ptr(x, torch.bfloat16, (T, H), "x"), T,
           _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
           _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(cw),
           _ptr(out, torch.bfloat16, (T, H), "out"), _ptr(ws, torch.uint8, None, "ws"),
           ws.numel(), _stream(), ev), "moe_forward_fused" if fused else "moe_forward")


def forward_noalloc(cfg: Config, x, topk_ids, topk_w, weights, out) -> None:
    """moe_forward_noalloc: moe_forward with the library's per-device scratch
    buffer as its workspace (no workspace argument, nothing allocated)."""
    import torch
    T = x.shape[0]
    H, k = cfg.hidden, cfg.top_k
    cw = weights if isinstance(weights, CWeights) else weights_struct(cfg, weights)
    cc = cfg.c()
    _ok(load().moe_forward_noalloc(ctypes.byref(cc), _ptr(x, torch.bfloat16, (T, H), "x"), T,
                                   _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                                   _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(cw),
                                   _ptr(out, torch.bfloat16, (T, H), "out"), _stream()), "moe_forward_noalloc")


def noalloc_scratch_bytes() -> int:
    return int(load().moe_noalloc_scratch_bytes())


def route_forward(cfg: Config, x, w_router, bias, topk_ids, topk_w, near_tie, weights, out, ws, events=None) -> None:
    """moe_route_forward: routing and the forward in one call; for small
    batches routing, x quantization and dispatch are one launch."""
    import torch
    T = x.shape[0]
    H, E, k = cfg.hidden, cfg.num_experts, cfg.top_k
    cw = weights if isinstance(weights, CWeights) else weights_struct(cfg, weights)
    ev = None
    if events is not None:
        if len(events) != 2 * len(STAGES):
            raise ValueError("events must hold 2 per stage")
        ev = (ctypes.c_void_p * len(events))(*[e.cuda_event if e is not None else None for e in events])
    cc = cfg.c()
    _ok(load().moe_route_forward(ctypes.byref(cc), _ptr(x, torch.bfloat16, (T, H), "x"), T,
                                 _ptr(w_router, torch.bfloat16, (E, H), "w_router"),
                                 _ptr(bias, torch.float32, (E,), "bias"),
                                 _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                                 _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                                 _ptr(near_tie, torch.uint8, (T,), "near_tie"), ctypes.byref(cw),
                                 _ptr(out, torch.bfloat16, (T, H), "out"), _ptr(ws, torch.uint8, None, "ws"),
                                 ws.numel(), _stream(), ev), "moe_route_forward")
