"""The C-ABI library without a GPU: it loads, exports every function that
include/moe.h declares, and its host-side checks reject bad arguments with
the documented status codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

import mixture_experts_forward_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced by host checks


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = moe.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.EXPORTS)


def test_status_strings():
    for s in range(6):
        assert moe.status_string(s)


def test_route_slots_formula():
    assert moe.route_slots(16, 2, 8, 16) == 160
    assert moe.route_slots(8, 8, 32, 16) == 544
    assert moe.route_slots(4096, 8, 32, 64) == 34816
    assert moe.route_slots(512, 8, 128, 32) == 8064
    assert moe.route_slots(65536, 8, 32, 256) == 532480
    assert moe.route_slots(0, 8, 32, 64) == 0


def test_plan_init_checks():
    L = moe.lib()
    p = moe.Plan()
    n = L.moe_plan_workspace_size(64, 8, 32, 16)
    assert n > 0
    assert L.moe_plan_init(ctypes.byref(p), FAKE, n, 64, 8, 32, 16) == OK
    assert p.route_slots == moe.route_slots(64, 8, 32, 16) and p.max_tiles == p.route_slots // 16
    assert L.moe_plan_init(ctypes.byref(p), FAKE, n - 1, 64, 8, 32, 16) == WORKSPACE
    assert L.moe_plan_init(ctypes.byref(p), ctypes.c_void_p(0x10010), n, 64, 8, 32, 16) == WORKSPACE
    assert L.moe_plan_init(ctypes.byref(p), FAKE, n, 64, 8, 32, 24) == UNSUPPORTED      # tile not a power of two
    assert L.moe_plan_init(ctypes.byref(p), FAKE, n, 64, 8, 32, 512) == UNSUPPORTED
    assert L.moe_plan_init(ctypes.byref(p), FAKE, n, 64, 0, 32, 16) == INVALID
    assert L.moe_plan_init(None, FAKE, n, 64, 8, 32, 16) == INVALID


def _plan(M=64, k=8, El=32, tile=16):
    p = moe.Plan()
    n = moe.lib().moe_plan_workspace_size(M, k, El, tile)
    assert moe.lib().moe_plan_init(ctypes.byref(p), FAKE, n, M, k, El, tile) == OK
    return p


def test_sort_argument_checks():
    L = moe.lib()
    p = _plan()
    assert L.moe_sort(FAKE, 64, 8, 256, 32, 240, 0, ctypes.byref(p), None) == INVALID   # offset + E_l > E
    assert L.moe_sort(FAKE, 63, 8, 256, 32, 0, 0, ctypes.byref(p), None) == INVALID     # M differs from the plan
    assert L.moe_sort(None, 64, 8, 256, 32, 0, 0, ctypes.byref(p), None) == INVALID
    assert L.moe_sort(FAKE, 64, 8, 256, 32, 0, 7, ctypes.byref(p), None) == INVALID     # route order
    assert L.moe_sort(FAKE, 64, 8, 256, 32, 0, 0, None, None) == INVALID


def test_gemm_argument_checks():
    L = moe.lib()
    p = ctypes.byref(_plan())
    g1 = L.moe_grouped_gemm1_swiglu
    F = FAKE
    # x_sf must be NULL exactly in W4A16; fc2_input_scale exactly in W4A4
    assert g1(0, F, F, 0, p, F, F, F, 256, 512, 1.0, 0.0, 1e30, None, F, None, None) == INVALID
    assert g1(1, F, F, 0, p, F, F, F, 256, 512, 1.0, 0.0, 1e30, None, F, F, None) == INVALID
    assert g1(2, F, F, 0, p, F, F, F, 256, 512, 1.0, 0.0, 1e30, F, F, F, None) == INVALID
    # H and I: multiples of the NVFP4 block (16) else invalid, of 32 else unsupported
    assert g1(0, F, None, 0, p, F, F, F, 200, 512, 1.0, 0.0, 1e30, None, F, None, None) == INVALID
    assert g1(0, F, None, 0, p, F, F, F, 208, 512, 1.0, 0.0, 1e30, None, F, None, None) == UNSUPPORTED
    assert g1(0, F, None, 0, p, F, F, F, 256, 80, 1.0, 0.0, 1e30, None, F, None, None) == UNSUPPORTED
    assert g1(2, F, F, 0, p, F, F, F, 256, 48, 1.0, 0.0, 1e30, None, F, F, None) == INVALID  # MX block 32
    assert g1(5, F, None, 0, p, F, F, F, 256, 512, 1.0, 0.0, 1e30, None, F, None, None) == INVALID
    assert g1(0, F, None, 100, p, F, F, F, 256, 512, 1.0, 0.0, 1e30, None, F, None, None) == INVALID  # stride < H
    g2 = L.moe_grouped_gemm2
    assert g2(0, F, None, p, F, F, F, 256, 512, F, None, 1.0, F, None) == INVALID   # both y2 and out
    assert g2(0, F, None, p, F, F, F, 256, 512, None, None, 1.0, None, None) == INVALID
    assert g2(0, F, None, p, F, F, F, 256, 512, None, None, 1.0, F, None) == INVALID  # atomic needs weights
    assert L.moe_finalize(F, p, F, 100, 1.0, 0, F, None) == UNSUPPORTED
    # alignment: y2 rows take 16-byte stores, out packed-bf16 atomics (4 bytes)
    # and, in the finalize, 16-byte accesses
    odd2, odd4 = ctypes.c_void_p(0x10002), ctypes.c_void_p(0x10004)
    assert g2(0, F, None, p, F, F, F, 256, 512, odd4, None, 1.0, None, None) == UNSUPPORTED
    assert g2(0, F, None, p, F, F, F, 256, 512, None, F, 1.0, odd2, None) == UNSUPPORTED
    assert L.moe_finalize(odd4, p, F, 256, 1.0, 0, F, None) == UNSUPPORTED
    assert L.moe_finalize(F, p, F, 256, 1.0, 0, odd4, None) == UNSUPPORTED


def test_activation_argument_checks():
    """The FC1 activation rules are checked on the host, before any launch."""
    L = moe.lib()
    p = ctypes.byref(_plan())
    F = FAKE
    g = lambda act, a=1.0, b=0.0, lim=moe.FLT_MAX, sb=0.0, slb=0.0, pts=None: L.moe_grouped_gemm1_act(
        0, F, None, 0, p, F, F, F, None, 256, 512, act, a, b, lim, sb, slb, None, pts, None, F, None, None)
    assert g(moe.ACT_RELU2, a=1.702) == INVALID                    # ReLU^2 takes no SwiGLU parameters
    assert g(moe.ACT_RELU2, sb=0.5) == INVALID                     # ... nor SiTU ones
    assert L.moe_grouped_gemm1_act(0, F, None, 0, p, F, F, F, F, 256, 512, moe.ACT_RELU2, 1.0, 0.0, moe.FLT_MAX,
                                   0.0, 0.0, None, None, None, F, None, None) == INVALID  # no up half to scale
    assert g(7) == INVALID                                         # unknown activation
    assert g(moe.ACT_GEGLU_TANH, a=1.702) == INVALID               # GeGLU takes no SwiGLU parameters
    assert g(moe.ACT_GEGLU_TANH, lim=7.0) == INVALID
    assert g(moe.ACT_GEGLU_TANH, sb=0.5) == INVALID                # ... nor SiTU ones
    assert g(moe.ACT_SWIGLU, sb=0.5, b=1.0) == INVALID             # SiTU with SwiGLU parameters
    assert g(moe.ACT_SWIGLU, slb=0.5) == INVALID                   # up clamp without SiTU
    assert g(moe.ACT_SWIGLU, sb=-1.0) == INVALID
    assert g(moe.ACT_SWIGLU, sb=float("inf")) == INVALID
    assert g(moe.ACT_SWIGLU, sb=float("nan")) == INVALID
    assert g(moe.ACT_SWIGLU, sb=0.5, slb=-0.1) == INVALID
    assert g(moe.ACT_SWIGLU, lim=0.0) == INVALID
    assert g(moe.ACT_SWIGLU, pts=F) == INVALID                     # per-token scales are W4A4 only
    # the forward checks the same rules before it enqueues anything
    o = moe.make_opts(activation=7)
    o.workspace = 0x10000
    o.workspace_bytes = 1 << 30
    args = (F, None, F, F, F, F, F, F, F, F, 8, 2, 8, 0, 0, F, 16, 256, 512, ctypes.byref(o), None)
    assert L.moe_forward(*args) == INVALID
    o.activation = moe.ACT_GEGLU_TANH
    o.swiglu_limit = 7.0
    assert L.moe_forward(*args) == INVALID


def test_forward_argument_checks():
    L = moe.lib()
    F = FAKE
    o = moe.make_opts()
    o.workspace = 0x10000
    o.workspace_bytes = 16
    args = lambda mode, xsf, M=16, H=256, I=512, El=8, off=0, E=8: (
        F, xsf, F, F, F, F, F, F, F, F, E, 2, El, off, mode, F, M, H, I, ctypes.byref(o), None)
    assert L.moe_forward(*args(0, None)) == WORKSPACE
    assert L.moe_forward(*args(0, F)) == INVALID
    assert L.moe_forward(*args(0, None, off=4)) == INVALID
    assert L.moe_forward(*args(0, None, H=300)) == INVALID       # not a multiple of the block
    assert L.moe_forward(*args(0, None, H=304)) == UNSUPPORTED   # a multiple of 16, not of 32
    assert L.moe_forward(*args(1, F)) == INVALID                 # W4A4 needs fc2_input_scale
    o.finalize_mode = 3
    assert L.moe_forward(*args(0, None)) == INVALID
    o.finalize_mode = 0
    o.path = 3
    assert L.moe_forward(*args(0, None)) == INVALID
    o.path = moe.PATH_AUTO
    # an output that is not 16-byte aligned
    odd = ctypes.c_void_p(0x10002)
    assert L.moe_forward(F, None, F, F, F, F, F, F, F, F, 8, 2, 8, 0, 0, odd, 16, 256, 512, ctypes.byref(o),
                         None) == UNSUPPORTED
    assert L.moe_forward(F, None, F, F, F, F, F, F, F, F, 8, 2, 8, 0, 0, F, 16, 256, 512, None, None) == INVALID


def test_forward_noalloc_host_checks():
    """moe_forward_noalloc takes no workspace and refuses, before anything
    is enqueued, a pass larger than its scratch array."""
    L = moe.lib()
    F = FAKE
    o = moe.make_opts()
    ws_opts = moe.make_opts()
    ws_opts.workspace = 0x10000
    ws_opts.workspace_bytes = 1 << 20
    args = lambda opts, M=8, H=6144, I=2048, E=256, El=32, k=8: (
        F, None, F, F, F, F, F, F, F, F, E, k, El, 0, 0, F, M, H, I, ctypes.byref(opts), None)
    assert L.moe_forward_noalloc(*args(ws_opts)) == INVALID
    assert L.moe_forward_noalloc(F, None, F, F, F, F, F, F, F, F, 256, 8, 32, 0, 0, F, 8, 6144, 2048, None,
                                 None) == INVALID
    # the prefill workload needs far more than 64 MiB of workspace
    need = moe.workspace_size(4096, 6144, 2048, 8, 32, 128, 0)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(*args(o, M=4096)) == 5
    assert "scratch" in moe.status_string(5)
    # the decode workload fits
    assert moe.workspace_size(8, 6144, 2048, 8, 32, 16, 0) <= moe.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_workspace_size_grows_with_mode():
    a = moe.workspace_size(16, 256, 512, 2, 8, 16, 0, 0)
    b = moe.workspace_size(16, 256, 512, 2, 8, 16, 0, 1)   # atomic: no y2
    c = moe.workspace_size(16, 256, 512, 2, 8, 16, 1, 0)   # NVFP4 y1 is smaller than bf16
    assert a > b > 0 and a > c > 0


def test_default_tile_counts_local_routes():
    """The tile rule estimates routes per local expert from the local share of
    the routes (M * top_k * E_l / E over E_l experts), not from all routes."""
    assert moe.default_tile(8, 8, 256, 32, 0) == 16          # decode: 0.25 routes per expert
    assert moe.default_tile(16, 2, 8, 8, 0) == 16            # tiny: 4
    assert moe.default_tile(512, 8, 128, 128, 1) == 32       # W4A4: 32
    assert moe.default_tile(4096, 8, 256, 32, 0) == 128      # prefill: 128
    assert moe.default_tile(65536, 8, 256, 32, 2) == 256     # MX large batch: 2048, the 256-slot kernel
    assert moe.default_tile(65536, 8, 256, 32, 0) == 128     # the same batch in W4A16
    assert moe.default_tile(12288, 8, 256, 32, 2) == 128     # MX at 384 routes per expert
    # the same batch over 8x the global experts puts 1/8 of the routes here
    assert moe.default_tile(1024, 8, 64, 8, 0) == 128        # 128 per expert
    assert moe.default_tile(1024, 8, 512, 8, 0) == 16        # 16 per expert
    assert moe.default_tile(1024, 8, 256, 8, 0) == 32        # 32 per expert
    assert moe.default_tile(1024, 8, 128, 8, 0) == 128       # 64 per expert: W4A16 goes wide
    assert moe.default_tile(1024, 8, 128, 8, 2) == 64        # MX at 64 per expert
    # W4A4 keeps the expert-streaming kernel's tiles at every larger size
    assert moe.default_tile(1024, 8, 128, 128, 1) == 64      # 64 per expert
    assert moe.default_tile(8192, 8, 128, 128, 1) == 64      # 512 per expert


def test_header_constants_match_binding():
    """The constants moe.h defines are the binding's."""
    import re
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(MOE_\w+)\s+(\d+)", text))
    assert int(consts["MOE_NUM_PHASE_EVENTS"]) == moe.NUM_PHASE_EVENTS
    enums = {k: int(v) for k, v in re.findall(r"\b(MOE_[A-Z0-9_]+)\s*=\s*(\d+)", text)}
    binding = {"MOE_QUANT_W4A16": moe.W4A16, "MOE_QUANT_W4A4": moe.W4A4, "MOE_QUANT_MXFP8_MXFP4": moe.MXFP8_MXFP4,
               "MOE_FINALIZE_DETERMINISTIC": moe.FINALIZE_DETERMINISTIC, "MOE_FINALIZE_ATOMIC": moe.FINALIZE_ATOMIC,
               "MOE_ROUTE_ORDER_AUTO": moe.ROUTE_ORDER_AUTO, "MOE_ROUTE_ORDER_SINGLE": moe.ROUTE_ORDER_SINGLE,
               "MOE_ROUTE_ORDER_SPAN": moe.ROUTE_ORDER_SPAN, "MOE_PATH_AUTO": moe.PATH_AUTO,
               "MOE_PATH_DECODE": moe.PATH_DECODE, "MOE_PATH_TILED": moe.PATH_TILED,
               "MOE_ACT_SWIGLU": moe.ACT_SWIGLU, "MOE_ACT_GEGLU_TANH": moe.ACT_GEGLU_TANH,
               "MOE_ACT_RELU2": moe.ACT_RELU2, "MOE_OK": moe.OK, "MOE_ERR_INVALID_ARGUMENT": moe.ERR_INVALID_ARGUMENT,
               "MOE_ERR_UNSUPPORTED": moe.ERR_UNSUPPORTED, "MOE_ERR_WORKSPACE": moe.ERR_WORKSPACE,
               "MOE_ERR_DEVICE": moe.ERR_DEVICE, "MOE_ERR_SCRATCH_TOO_SMALL": moe.ERR_SCRATCH_TOO_SMALL}
    for name, value in binding.items():
        assert enums[name] == value, name


def test_forward_plan_view():
    """moe_forward_plan carves the plan at a fixed place inside a forward
    workspace: after the counter block, inside the workspace, with the
    capacity of a plan of the same shape, and rejects a short workspace."""
    L = moe.lib()
    for (M, H, I, k, El, tile, mode) in [(8, 6144, 2048, 8, 32, 16, 0), (4096, 6144, 2048, 8, 32, 128, 0),
                                         (16, 256, 512, 2, 8, 16, 1), (512, 4096, 1536, 8, 128, 32, 2)]:
        n = moe.workspace_size(M, H, I, k, El, tile, mode)
        pn = L.moe_plan_workspace_size(M, k, El, tile)
        p = moe.Plan()
        assert L.moe_forward_plan(ctypes.byref(p), FAKE, n, M, k, El, tile) == OK
        base = FAKE.value
        assert p.expanded_to_permuted % 256 == 0 and p.expanded_to_permuted > base
        assert p.scratch - base < n and p.route_slots == moe.route_slots(M, k, El, tile)
        assert p.expanded_to_permuted - base + pn <= n
        assert L.moe_forward_plan(ctypes.byref(p), FAKE, p.expanded_to_permuted - base + pn - 1, M, k, El,
                                  tile) == WORKSPACE
        assert L.moe_forward_plan(ctypes.byref(p), None, n, M, k, El, tile) == WORKSPACE
        assert L.moe_forward_plan(None, FAKE, n, M, k, El, tile) == INVALID


def test_forward_accepts_the_workspace_it_asks_for():
    """moe_forward's host checks accept exactly moe_workspace_size() bytes
    for every launch sequence (decode path included) and reject one byte
    less.  Run without a GPU, so the call stops at the first device step
    with MOE_ERR_DEVICE instead of launching on placeholder pointers."""
    import ctypes

    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must not reach a launch on a machine with a GPU")
    L = moe.lib()
    buf = torch.zeros(1 << 20, dtype=torch.uint8)
    P = ctypes.c_void_p(buf.data_ptr())
    for (M, H, I, E, El, k, tile) in [(6, 2048, 512, 64, 8, 4, 16), (8, 6144, 2048, 256, 32, 8, 16),
                                      (40, 256, 256, 8, 8, 2, 16), (37, 384, 256, 16, 6, 4, 64)]:
        for fm in (moe.FINALIZE_DETERMINISTIC, moe.FINALIZE_ATOMIC):
            n = moe.workspace_size(M, H, I, k, El, tile, 0, fm)
            ws = torch.zeros(n + 512, dtype=torch.uint8)
            for size, want_ws_error in ((n, False), (n - 1, True)):
                o = moe.make_opts(tile=tile, finalize_mode=fm)
                o.workspace = ws.data_ptr() + (-ws.data_ptr()) % 256
                o.workspace_bytes = size
                st = L.moe_forward(P, None, P, P, P, P, P, P, P, P, E, k, El, 0, 0, P, M, H, I, ctypes.byref(o), None)
                assert (st == 3) == want_ws_error, (M, H, I, tile, fm, size, st)
