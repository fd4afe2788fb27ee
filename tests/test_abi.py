"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and the host-side argument checks return the
documented statuses before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

import block_scaled_expert_amd as bse

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bse.LIB_PATH):
        from block_scaled_expert_amd import build
        build.build()
    return bse.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_quantize_act", "moe_forward", "moe_forward_fused", "moe_dispatch",
              "moe_prepare_weights", "moe_workspace_size", "moe_status_string", "moe_check_arch",
              "moe_validate_config", "moe_encode_weights", "moe_decode_weights", "moe_forward_fused_status",
              "moe_cap_swiglu", "moe_forward_noalloc", "moe_noalloc_scratch_bytes"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", bse.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(moe_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(bse.EXPORTED) <= exported


def test_check_arch(lib):
    assert bse.check_arch("gfx950") == 0
    assert bse.check_arch("gfx950:sramecc+:xnack-") == 0
    for bad in ("gfx942", "gfx9500", "gfx90a", "", "gfx95"):
        assert bse.check_arch(bad) == -2, bad
    assert lib.moe_check_arch(None) == -1


def test_status_strings(lib):
    for st in range(0, -9, -1):
        assert bse.status_string(st) != "unknown status"
    assert bse.status_string(-99) == "unknown status"


def _cfg(**kw):
    base = dict(hidden=4608, ffn=2304, num_experts=384, top_k=8, fmt="nvfp4", max_tokens=64)
    base.update(kw)
    return bse.Config(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"hidden": 4600}, -1), ({"ffn": 100}, -1), ({"num_experts": 0}, -1), ({"num_experts": 2000}, -1),
    ({"top_k": 0}, -1), ({"top_k": 33}, -1), ({"num_experts": 4, "top_k": 5}, -1),
    ({"expert_begin": 380, "num_local_experts": 8}, -1), ({"num_local_experts": 0}, -1),
    ({"cap_form": 7}, -1), ({"cap": 0.0}, -1), ({"cap": 0.0, "cap_form": 3}, 0),
    ({"max_tokens": -1}, -1), ({"max_tokens": 1 << 22}, -1),
])
def test_validate_config(lib, kw, status):
    cc = _cfg(**kw).c()
    assert lib.moe_validate_config(ctypes.byref(cc)) == status


def test_unsupported_format(lib):
    cc = _cfg().c()
    cc.fmt = 3
    assert lib.moe_validate_config(ctypes.byref(cc)) == -5


def test_workspace_size_grows_with_tokens(lib):
    sizes = [bse.workspace_size(_cfg(max_tokens=t)) for t in (0, 1, 64, 192, 16384)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    # the fp32 SwiGLU output and expert outputs dominate: P*(F+H)*4 bytes
    assert sizes[-1] >= 16384 * 8 * (2304 + 4608) * 4


def test_host_checks_before_device(lib):
    """Argument errors come back without a GPU (nothing is enqueued)."""
    cc = _cfg(max_tokens=64).c()
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(cc), None) == -1
    assert lib.moe_workspace_size(ctypes.byref(cc), ctypes.byref(n)) == 0
    # too many tokens
    assert lib.moe_route(ctypes.byref(cc), None, 65, None, None, None, None, None, None, 0, None) == -4
    assert lib.moe_forward(ctypes.byref(cc), None, 65, None, None, None, None, None, 0, None, None) == -4
    # null / misaligned / small workspace
    assert lib.moe_route(ctypes.byref(cc), None, 8, None, None, None, None, None, None, 0, None) == -1
    assert lib.moe_forward(ctypes.byref(cc), None, 8, None, None, None, None, ctypes.c_void_p(0x1001),
                           n.value, None, None) == -1
    assert lib.moe_forward(ctypes.byref(cc), None, 8, None, None, None, None, ctypes.c_void_p(0x1000),
                           n.value - 1, None, None) == -3
    assert lib.moe_dispatch(ctypes.byref(cc), None, 8, None, None, None, ctypes.c_void_p(0x1000), n.value,
                            None) == -1
    # zero tokens is a no-op that needs no device
    assert lib.moe_forward(ctypes.byref(cc), None, 0, None, None, None, None, ctypes.c_void_p(0x1000), n.value,
                           None, None) == 0
    # the single-launch variant checks its arguments the same way
    assert lib.moe_forward_fused(ctypes.byref(cc), None, 65, None, None, None, None, None, 0, None, None) == -4
    assert lib.moe_forward_fused(ctypes.byref(cc), None, 8, None, None, None, None, ctypes.c_void_p(0x1001),
                                 n.value, None, None) == -1
    assert lib.moe_forward_fused(ctypes.byref(cc), None, 8, None, None, None, None, ctypes.c_void_p(0x1000),
                                 n.value - 1, None, None) == -3
    assert lib.moe_forward_fused(ctypes.byref(cc), None, 0, None, None, None, None, ctypes.c_void_p(0x1000),
                                 n.value, None, None) == 0
    # bad quantize arguments
    q = lib.moe_quantize_act
    r = ctypes.byref(cc)
    assert q(r, 0, 0, None, 4, 48, None, None, None, None, 0, None) == -1   # cols % 32
    bad = _cfg().c()
    bad.fmt = 3
    assert q(ctypes.byref(bad), 0, 0, None, 4, 64, None, None, None, None, 0, None) == -5   # format
    assert q(r, 0, 2, None, 4, 64, None, None, None, None, 0, None) == -1   # dtype
    assert q(r, 2, 0, None, 4, 64, None, None, None, None, 0, None) == -1   # site
    assert q(r, 0, 0, None, 0, 64, None, None, None, None, 0, None) == 0    # nothing to do
    # weights: bad layout value / canonical source required
    w = bse.CWeights(1, 1, 1, 1, 1, 5)
    assert lib.moe_prepare_weights(ctypes.byref(cc), ctypes.byref(w), ctypes.byref(bse.CWeights()), None) == -1


def test_encode_decode_host_checks(lib):
    """Weight encoder / decoder argument errors come back without a GPU."""
    p = ctypes.c_void_p(0x1000)
    enc, dec = lib.moe_encode_weights, lib.moe_decode_weights
    assert enc(3, 0, p, 2, 16, 64, p, p, p, 1, 1, p, 64, None) == -5        # format
    assert enc(1, 2, p, 2, 16, 64, p, p, p, 1, 1, p, 64, None) == -1        # dtype
    assert enc(1, 0, p, 2, 16, 48, p, p, p, 1, 1, p, 64, None) == -1        # cols % 32
    assert enc(1, 0, p, 0, 16, 64, None, None, None, 1, 1, None, 0, None) == 0   # nothing to do
    assert enc(1, 0, None, 2, 16, 64, p, p, p, 1, 1, p, 64, None) == -1     # null input
    assert enc(1, 0, ctypes.c_void_p(0x1008), 2, 16, 64, p, p, p, 1, 1, p, 64, None) == -1   # alignment
    assert enc(1, 0, p, 2, 16, 64, p, p, None, 1, 1, p, 64, None) == -1     # NVFP4 needs gs
    assert enc(1, 0, p, 2, 16, 64, p, p, p, 2, 1, p, 64, None) == -1        # stride < group
    assert enc(1, 0, p, 4, 16, 64, p, p, p, 1, 1, p, 15, None) == -3        # scratch for 4 maxima
    assert dec(3, p, p, p, 1, 1, 2, 16, 64, p, None) == -5
    assert dec(1, p, p, None, 1, 1, 2, 16, 64, p, None) == -1
    assert dec(2, p, p, None, 1, 1, 0, 16, 64, p, None) == 0


def test_act_gs_config(lib):
    for kw, status in [({"act_gs": 0}, 0), ({"act_gs": 1}, 0), ({"act_gs": 2}, 0), ({"act_gs": 3}, -1),
                       ({"act_gs": -1}, -1), ({"act_gs": 2, "act_gs_static": (0.0, 1.0)}, -1),
                       ({"act_gs": 2, "act_gs_static": (1.0, float("nan"))}, -1),
                       ({"act_gs": 2, "act_gs_static": (1.0, float("inf"))}, -1),
                       ({"act_gs": 2, "act_gs_static": (1.0, 2.0 ** 121)}, -1),
                       ({"act_gs": 2, "act_gs_static": (2.0 ** -100, 2.0 ** 120)}, 0),
                       # MXFP8 carries no fp32 activation scale: the static values are not read
                       ({"fmt": "mxfp8", "act_gs": 2, "act_gs_static": (0.0, 0.0)}, 0)]:
        cc = _cfg(**kw).c()
        assert lib.moe_validate_config(ctypes.byref(cc)) == status, kw
    # per-tensor NVFP4 needs scratch for its two passes; the others do not
    q = lib.moe_quantize_act
    p = ctypes.c_void_p(0x1000)
    cc = _cfg(act_gs=1).c()
    assert q(ctypes.byref(cc), 0, 0, p, 4, 64, p, p, p, None, 0, None) == -1
    assert q(ctypes.byref(cc), 0, 0, p, 4, 64, p, p, p, p, bse.ACT_GS_SCRATCH_BYTES - 1, None) == -3


MISALIGNED = ctypes.c_void_p(0x1008)   # 8-byte aligned, not 16


def test_alignment_checked_before_device(lib):
    """Pointers the kernels read or write with 16-byte vector accesses are
    rejected when misaligned, before anything is enqueued."""
    cc = _cfg(max_tokens=64).c()
    r = ctypes.byref(cc)
    n = ctypes.c_size_t(0)
    lib.moe_workspace_size(r, ctypes.byref(n))
    ws, ok = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x2000)
    # moe_quantize_act: x and codes 16-byte aligned, row_gs 4
    q = lib.moe_quantize_act
    assert q(r, 0, 0, MISALIGNED, 4, 64, ok, ok, ok, None, 0, None) == -1
    assert q(r, 0, 0, ok, 4, 64, MISALIGNED, ok, ok, None, 0, None) == -1
    assert q(r, 0, 0, ok, 4, 64, ok, ok, ctypes.c_void_p(0x2002), None, 0, None) == -1
    # moe_route: x and the router weight 16, bias / ids / weights 4
    rt = lib.moe_route
    assert rt(r, MISALIGNED, 8, ok, ok, ok, ok, None, ws, n.value, None) == -1
    assert rt(r, ok, 8, MISALIGNED, ok, ok, ok, None, ws, n.value, None) == -1
    assert rt(r, ok, 8, ok, ctypes.c_void_p(0x2001), ok, ok, None, ws, n.value, None) == -1
    # moe_forward / moe_forward_fused: x, out, w13, w2 16; scales, gs, ids, weights 4
    good = bse.CWeights(0x4000, 0x5000, 0x6000, 0x7000, 0x8000, 1)
    for fwd in (lib.moe_forward, lib.moe_forward_fused):
        assert fwd(r, MISALIGNED, 8, ok, ok, ctypes.byref(good), ok, ws, n.value, None, None) == -1
        assert fwd(r, ok, 8, ok, ok, ctypes.byref(good), MISALIGNED, ws, n.value, None, None) == -1
        assert fwd(r, ok, 8, ctypes.c_void_p(0x2002), ok, ctypes.byref(good), ok, ws, n.value, None, None) == -1
        for field, bad_ptr in (("w13", 0x4008), ("w2", 0x6008), ("w13_sc", 0x5002), ("w2_sc", 0x7001),
                               ("gs", 0x8002)):
            w = bse.CWeights(0x4000, 0x5000, 0x6000, 0x7000, 0x8000, 1)
            setattr(w, field, bad_ptr)
            assert fwd(r, ok, 8, ok, ok, ctypes.byref(w), ok, ws, n.value, None, None) == -1, field
    # moe_cap_swiglu and moe_forward_fused_status: 4-byte aligned arrays
    assert lib.moe_cap_swiglu(r, ctypes.c_void_p(0x2002), ok, 16, ok, None) == -1
    assert lib.moe_cap_swiglu(r, ok, ok, -1, ok, None) == -1
    assert lib.moe_cap_swiglu(r, None, None, 0, None, None) == 0
    assert lib.moe_forward_fused_status(r, 8, ws, n.value, ctypes.c_void_p(0x2002), None) == -1
    assert lib.moe_forward_fused_status(r, 8, ws, n.value - 1, ok, None) == -3
    assert lib.moe_forward_fused_status(r, 65, ws, n.value, ok, None) == -4


def test_noalloc_host_checks(lib):
    """moe_forward_noalloc rejects, before touching a device, a batch whose
    workspace exceeds its fixed 64 MiB buffer, and T above max_tokens."""
    assert lib.moe_noalloc_scratch_bytes() == 64 << 20
    big = _cfg(max_tokens=1024).c()
    assert lib.moe_forward_noalloc(ctypes.byref(big), None, 270, None, None, None, None, None) == -8
    assert lib.moe_forward_noalloc(ctypes.byref(big), None, 1025, None, None, None, None, None) == -4
    assert lib.moe_forward_noalloc(ctypes.byref(big), None, 0, None, None, None, None, None) == 0
    assert lib.moe_forward_noalloc(ctypes.byref(big), None, -1, None, None, None, None, None) == -1
    assert "64 MiB" in bse.status_string(-8)
