"""Python binding of libmoe_mi355x.so, the MI355X (gfx950) fused MoE forward.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/moe.h.  torch provides device
memory and the current stream.  There is no fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

W4A16, W4A4, MXFP8_MXFP4 = 0, 1, 2
FINALIZE_DETERMINISTIC, FINALIZE_ATOMIC = 0, 1
ROUTE_ORDER_AUTO, ROUTE_ORDER_SINGLE, ROUTE_ORDER_SPAN = 0, 1, 2
PATH_AUTO, PATH_DECODE, PATH_TILED = 0, 1, 2   # moe_path_t
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE, ERR_SCRATCH_TOO_SMALL = range(6)  # moe_status_t
NUM_PHASE_EVENTS = 5
FLT_MAX = 3.4028234663852886e38
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
ACT_SWIGLU, ACT_GEGLU_TANH, ACT_RELU2 = 0, 1, 2   # moe_activation_t (SiTU: ACT_SWIGLU with situ_beta > 0)

EXPORTS = [
    "moe_status_string", "moe_route_slots", "moe_plan_workspace_size", "moe_plan_init", "moe_sort",
    "moe_grouped_gemm1_swiglu", "moe_grouped_gemm1_act", "moe_grouped_gemm2", "moe_grouped_gemm2_bias", "moe_finalize", "moe_opts_init", "moe_default_tile",
    "moe_workspace_size", "moe_forward_plan", "moe_forward", "moe_forward_noalloc", "moe_fc2_input_scale", "moe_nvfp4_global_scale", "moe_quantize_nvfp4", "moe_quantize_mx",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [
        ("expanded_to_permuted", ctypes.c_void_p), ("permuted_to_expanded", ctypes.c_void_p),
        ("tile_to_expert", ctypes.c_void_p), ("tile_to_mn_limit", ctypes.c_void_p),
        ("num_tiles", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p), ("route_slots", ctypes.c_int64), ("max_tiles", ctypes.c_int32),
        ("tile", ctypes.c_int32), ("M", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("num_local_experts", ctypes.c_int32), ("max_spans", ctypes.c_int32),
    ]


class Opts(ctypes.Structure):
    _fields_ = [
        ("swiglu_alpha", ctypes.c_float), ("swiglu_beta", ctypes.c_float), ("swiglu_limit", ctypes.c_float),
        ("fc2_input_scale", ctypes.c_void_p), ("routed_scaling_factor", ctypes.c_float),
        ("accumulate", ctypes.c_int), ("finalize_mode", ctypes.c_int), ("route_order", ctypes.c_int),
        ("tile", ctypes.c_int), ("x_row_stride", ctypes.c_int64), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("phase_events", ctypes.c_void_p),
        ("activation", ctypes.c_int), ("situ_beta", ctypes.c_float), ("situ_linear_beta", ctypes.c_float),
        ("w1_alpha_up", ctypes.c_void_p), ("per_token_scale", ctypes.c_void_p),
        ("fc1_bias", ctypes.c_void_p), ("fc2_bias", ctypes.c_void_p), ("path", ctypes.c_int),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The native library.  Raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -m mixture_experts_forward_moe_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        sigs = {
            "moe_status_string": ([I], ctypes.c_char_p),
            "moe_route_slots": ([I, I, I, I], I64),
            "moe_plan_workspace_size": ([I, I, I, I], SZ),
            "moe_plan_init": ([P, P, SZ, I, I, I, I], I),
            "moe_sort": ([P, I, I, I, I, I, I, P, P], I),
            "moe_grouped_gemm1_swiglu": ([I, P, P, I64, P, P, P, P, I, I, F, F, F, P, P, P, P], I),
            "moe_grouped_gemm1_act": ([I, P, P, I64, P, P, P, P, P, I, I, I, F, F, F, F, F, P, P, P, P, P, P], I),
            "moe_grouped_gemm2_bias": ([I, P, P, P, P, P, P, P, I, I, P, P, F, P, P], I),
            "moe_grouped_gemm2": ([I, P, P, P, P, P, P, I, I, P, P, F, P, P], I),
            "moe_finalize": ([P, P, P, I, F, I, P, P], I),
            "moe_opts_init": ([P], None),
            "moe_default_tile": ([I, I, I, I, I], I),
            "moe_workspace_size": ([I, I, I, I, I, I, I, I], SZ),
            "moe_forward_plan": ([P, P, SZ, I, I, I, I], I),
            "moe_forward": ([P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, I, I, I, P, P], I),
            "moe_forward_noalloc": ([P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, I, I, I, P, P], I),
            "moe_fc2_input_scale": ([P, P, I64, P, P, P, P, P, I, I, I, F, F, F, F, F, P, P, P, P], I),
            "moe_nvfp4_global_scale": ([P, I64, I64, P, P], I),
            "moe_quantize_nvfp4": ([P, I64, I64, I64, P, P, P, P], I),
            "moe_quantize_mx": ([P, I64, I64, I, P, P, P], I),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def _ptr(t):
    """device pointer of a tensor (or None)"""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def route_slots(M: int, top_k: int, num_local_experts: int, tile: int) -> int:
    return lib().moe_route_slots(M, top_k, num_local_experts, tile)


def default_tile(M: int, top_k: int, num_experts: int, num_local_experts: int, mode: int) -> int:
    return lib().moe_default_tile(M, top_k, num_experts, num_local_experts, mode)


def workspace_size(M, H, I, top_k, num_local_experts, tile, mode, finalize_mode=FINALIZE_DETERMINISTIC) -> int:
    return lib().moe_workspace_size(M, H, I, top_k, num_local_experts, tile, mode, finalize_mode)


def _alloc(nbytes: int, device):
    import torch
    # 256-byte alignment: torch's caching allocator aligns blocks to 512 bytes.
    # No initial contents are needed: every piece is written before it is read.
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


class MoePlan:
    """A routing plan with its device workspace (torch-owned).  With
    `forward_workspace`, a view of the plan a moe_forward built in that
    workspace (moe_forward_plan) instead of a workspace of its own."""

    def __init__(self, M: int, top_k: int, num_local_experts: int, tile: int, device="cuda",
                 forward_workspace=None):
        self.c = Plan()
        if forward_workspace is not None:
            self.workspace = forward_workspace
            _check(lib().moe_forward_plan(ctypes.byref(self.c), _ptr(forward_workspace), forward_workspace.numel(),
                                          M, top_k, num_local_experts, tile), "moe_forward_plan")
        else:
            n = lib().moe_plan_workspace_size(M, top_k, num_local_experts, tile)
            if n == 0:
                raise MoeError(1, "moe_plan_workspace_size")
            self.workspace = _alloc(n, device)
            _check(lib().moe_plan_init(ctypes.byref(self.c), _ptr(self.workspace), n, M, top_k, num_local_experts,
                                       tile), "moe_plan_init")
        self.M, self.top_k, self.num_local_experts, self.tile = M, top_k, num_local_experts, tile
        self.route_slots = self.c.route_slots
        self.max_tiles = self.c.max_tiles

    def _view(self, field, n):
        import torch
        off = getattr(self.c, field) - self.workspace.data_ptr()
        return self.workspace[off:off + 4 * n].view(torch.int32)

    @property
    def expanded_to_permuted(self):
        return self._view("expanded_to_permuted", self.M * self.top_k)

    @property
    def permuted_to_expanded(self):
        return self._view("permuted_to_expanded", self.route_slots)

    @property
    def tile_to_expert(self):
        return self._view("tile_to_expert", self.max_tiles)

    @property
    def tile_to_mn_limit(self):
        return self._view("tile_to_mn_limit", self.max_tiles)

    @property
    def num_tiles(self):
        return self._view("num_tiles", 1)

    @property
    def expert_offsets(self):
        return self._view("expert_offsets", self.num_local_experts + 1)

    @property
    def expert_counts(self):
        return self._view("expert_counts", self.num_local_experts)


def moe_sort(topk_ids, num_experts: int, num_local_experts: int, local_expert_offset: int, tile: int,
             route_order: int = ROUTE_ORDER_AUTO, plan: MoePlan | None = None, stream=None) -> MoePlan:
    M, top_k = topk_ids.shape
    if plan is None:
        plan = MoePlan(M, top_k, num_local_experts, tile, topk_ids.device)
    _check(lib().moe_sort(_ptr(topk_ids), M, top_k, num_experts, num_local_experts, local_expert_offset, route_order,
                          ctypes.byref(plan.c), _stream(stream)), "moe_sort")
    return plan


def moe_grouped_gemm1_swiglu(mode, x, x_sf, plan: MoePlan, w1, w1_sf, w1_alpha, H, I, y1, y1_sf=None,
                             swiglu_alpha=1.0, swiglu_beta=0.0, swiglu_limit=FLT_MAX, fc2_input_scale=None,
                             x_row_stride=0, stream=None):
    _check(lib().moe_grouped_gemm1_swiglu(mode, _ptr(x), _ptr(x_sf), x_row_stride, ctypes.byref(plan.c), _ptr(w1),
                                          _ptr(w1_sf), _ptr(w1_alpha), H, I, swiglu_alpha, swiglu_beta, swiglu_limit,
                                          _ptr(fc2_input_scale), _ptr(y1), _ptr(y1_sf), _stream(stream)),
           "moe_grouped_gemm1_swiglu")


def moe_grouped_gemm1_act(mode, x, x_sf, plan: MoePlan, w1, w1_sf, w1_alpha, H, I, y1, y1_sf=None,
                          activation=ACT_SWIGLU, swiglu_alpha=1.0, swiglu_beta=0.0, swiglu_limit=FLT_MAX,
                          situ_beta=0.0, situ_linear_beta=0.0, fc2_input_scale=None, x_row_stride=0, stream=None,
                          w1_alpha_up=None, per_token_scale=None, fc1_bias=None):
    _check(lib().moe_grouped_gemm1_act(mode, _ptr(x), _ptr(x_sf), x_row_stride, ctypes.byref(plan.c), _ptr(w1),
                                       _ptr(w1_sf), _ptr(w1_alpha), _ptr(w1_alpha_up), H, I, activation,
                                       swiglu_alpha, swiglu_beta, swiglu_limit, situ_beta, situ_linear_beta,
                                       _ptr(fc2_input_scale), _ptr(per_token_scale), _ptr(fc1_bias), _ptr(y1),
                                       _ptr(y1_sf),
                                       _stream(stream)), "moe_grouped_gemm1_act")


def moe_grouped_gemm2(mode, y1, y1_sf, plan: MoePlan, w2, w2_sf, w2_alpha, H, I, y2=None, topk_weights=None,
                      routed_scaling_factor=1.0, out=None, stream=None, fc2_bias=None):
    if fc2_bias is None:
        _check(lib().moe_grouped_gemm2(mode, _ptr(y1), _ptr(y1_sf), ctypes.byref(plan.c), _ptr(w2), _ptr(w2_sf),
                                       _ptr(w2_alpha), H, I, _ptr(y2), _ptr(topk_weights), routed_scaling_factor,
                                       _ptr(out), _stream(stream)), "moe_grouped_gemm2")
    else:
        _check(lib().moe_grouped_gemm2_bias(mode, _ptr(y1), _ptr(y1_sf), ctypes.byref(plan.c), _ptr(w2),
                                            _ptr(w2_sf), _ptr(w2_alpha), _ptr(fc2_bias), H, I, _ptr(y2),
                                            _ptr(topk_weights), routed_scaling_factor, _ptr(out), _stream(stream)),
               "moe_grouped_gemm2_bias")


def moe_finalize(y2, plan: MoePlan, topk_weights, H, out, routed_scaling_factor=1.0, accumulate=False, stream=None):
    _check(lib().moe_finalize(_ptr(y2), ctypes.byref(plan.c), _ptr(topk_weights), H, routed_scaling_factor,
                              int(bool(accumulate)), _ptr(out), _stream(stream)), "moe_finalize")


def make_opts(workspace=None, swiglu_alpha=1.0, swiglu_beta=0.0, swiglu_limit=FLT_MAX, fc2_input_scale=None,
              routed_scaling_factor=1.0, accumulate=False, finalize_mode=FINALIZE_DETERMINISTIC,
              route_order=ROUTE_ORDER_AUTO, tile=0, x_row_stride=0, phase_events=None, activation=ACT_SWIGLU,
              situ_beta=0.0, situ_linear_beta=0.0, w1_alpha_up=None, per_token_scale=None, fc1_bias=None,
              fc2_bias=None, path=PATH_AUTO) -> Opts:
    o = Opts()
    lib().moe_opts_init(ctypes.byref(o))
    o.swiglu_alpha, o.swiglu_beta, o.swiglu_limit = swiglu_alpha, swiglu_beta, swiglu_limit
    o.activation, o.situ_beta, o.situ_linear_beta = activation, situ_beta, situ_linear_beta
    o.w1_alpha_up = None if w1_alpha_up is None else w1_alpha_up.data_ptr()
    o.per_token_scale = None if per_token_scale is None else per_token_scale.data_ptr()
    o.fc1_bias = None if fc1_bias is None else fc1_bias.data_ptr()
    o.fc2_bias = None if fc2_bias is None else fc2_bias.data_ptr()
    o.fc2_input_scale = None if fc2_input_scale is None else fc2_input_scale.data_ptr()
    o.routed_scaling_factor = routed_scaling_factor
    o.accumulate = int(bool(accumulate))
    o.finalize_mode = finalize_mode
    o.route_order = route_order
    o.tile = tile
    o.x_row_stride = x_row_stride
    o.path = path
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    if phase_events is not None:
        arr = (ctypes.c_void_p * NUM_PHASE_EVENTS)(*[None if e is None else e.cuda_event for e in phase_events])
        o._events = arr
        o.phase_events = ctypes.cast(arr, ctypes.c_void_p)
    return o


def moe_forward(x, x_sf, topk_ids, topk_weights, w1, w1_sf, w1_alpha, w2, w2_sf, w2_alpha, num_experts: int,
                top_k: int, num_local_experts: int, local_expert_offset: int, quant_mode: int, out, H: int, I: int,
                opts: Opts | None = None, workspace=None, stream=None, **kw):
    """The whole forward pass into `out` (bf16 [M, H]).  A workspace is taken
    from `workspace`, or allocated here (outside the library) when None."""
    M = topk_ids.shape[0]
    if opts is None:
        tile = kw.pop("tile", 0) or default_tile(M, top_k, num_experts, num_local_experts, quant_mode)
        fm = kw.get("finalize_mode", FINALIZE_DETERMINISTIC)
        if workspace is None:
            workspace = _alloc(workspace_size(M, H, I, top_k, num_local_experts, tile, quant_mode, fm), x.device)
        opts = make_opts(workspace=workspace, tile=tile, **kw)
    _check(lib().moe_forward(_ptr(x), _ptr(x_sf), _ptr(topk_ids), _ptr(topk_weights), _ptr(w1), _ptr(w1_sf),
                             _ptr(w1_alpha), _ptr(w2), _ptr(w2_sf), _ptr(w2_alpha), num_experts, top_k,
                             num_local_experts, local_expert_offset, quant_mode, _ptr(out), M, H, I,
                             ctypes.byref(opts), _stream(stream)), "moe_forward")
    return out


def moe_forward_noalloc(x, x_sf, topk_ids, topk_weights, w1, w1_sf, w1_alpha, w2, w2_sf, w2_alpha, num_experts: int,
                        top_k: int, num_local_experts: int, local_expert_offset: int, quant_mode: int, out, H: int,
                        I: int, stream=None, **kw):
    """moe_forward with the library's own fixed scratch array as workspace
    (nothing is allocated, here or in the library)."""
    M = topk_ids.shape[0]
    opts = make_opts(**kw)
    _check(lib().moe_forward_noalloc(_ptr(x), _ptr(x_sf), _ptr(topk_ids), _ptr(topk_weights), _ptr(w1), _ptr(w1_sf),
                                     _ptr(w1_alpha), _ptr(w2), _ptr(w2_sf), _ptr(w2_alpha), num_experts, top_k,
                                     num_local_experts, local_expert_offset, quant_mode, _ptr(out), M, H, I,
                                     ctypes.byref(opts), _stream(stream)), "moe_forward_noalloc")
    return out


def moe_fc2_input_scale(x, x_sf, plan: MoePlan, w1, w1_sf, w1_alpha, H, I, fc2_input_scale, activation=ACT_SWIGLU,
                        swiglu_alpha=1.0, swiglu_beta=0.0, swiglu_limit=FLT_MAX, situ_beta=0.0, situ_linear_beta=0.0,
                        x_row_stride=0, w1_alpha_up=None, per_token_scale=None, fc1_bias=None, stream=None):
    """W4A4: fc2_input_scale (device fp32 [1]) = max |y1| / (6 * 448) over the plan's routes."""
    _check(lib().moe_fc2_input_scale(_ptr(x), _ptr(x_sf), x_row_stride, ctypes.byref(plan.c), _ptr(w1), _ptr(w1_sf),
                                     _ptr(w1_alpha), _ptr(w1_alpha_up), H, I, activation, swiglu_alpha, swiglu_beta,
                                     swiglu_limit, situ_beta, situ_linear_beta, _ptr(per_token_scale),
                                     _ptr(fc1_bias), _ptr(fc2_input_scale), _stream(stream)), "moe_fc2_input_scale")


def moe_nvfp4_global_scale(x, batches: int, gscale, stream=None):
    _check(lib().moe_nvfp4_global_scale(_ptr(x), batches, x.numel() // max(batches, 1), _ptr(gscale),
                                        _stream(stream)), "moe_nvfp4_global_scale")


def moe_quantize_nvfp4(x, batches: int, rows: int, cols: int, gscale, q, sf, stream=None):
    _check(lib().moe_quantize_nvfp4(_ptr(x), batches, rows, cols, _ptr(gscale), _ptr(q), _ptr(sf), _stream(stream)),
           "moe_quantize_nvfp4")


def moe_quantize_mx(x, rows: int, cols: int, elem: int, q, sf, stream=None):
    _check(lib().moe_quantize_mx(_ptr(x), rows, cols, elem, _ptr(q), _ptr(sf), _stream(stream)), "moe_quantize_mx")
