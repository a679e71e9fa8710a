"""CPU oracle of the fused MoE forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
fp64 sums) with numpy; it shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

W4A16, W4A4, MXFP8_MXFP4 = 0, 1, 2
ELEM_E4M3, ELEM_E2M1 = 0, 1
ACT_SWIGLU, ACT_GEGLU_TANH, ACT_RELU2 = 0, 1, 2   # FC1 activations (SiTU: SwiGLU with situ_beta > 0;
#                                                 ReLU^2 is non-gated, W1 has I rows)


def build(force: bool = True) -> str:
    """Compile liboracle.so (gcc -O2, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-D_GNU_SOURCE", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Moe(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int), ("M", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
        ("top_k", ctypes.c_int), ("num_experts", ctypes.c_int), ("num_local_experts", ctypes.c_int),
        ("local_expert_offset", ctypes.c_int),
        ("x", ctypes.c_void_p), ("x_sf", ctypes.c_void_p), ("x_row_stride", ctypes.c_int64),
        ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
        ("w1", ctypes.c_void_p), ("w1_sf", ctypes.c_void_p), ("w1_alpha", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p), ("w2_alpha", ctypes.c_void_p),
        ("swiglu_alpha", ctypes.c_float), ("swiglu_beta", ctypes.c_float), ("swiglu_limit", ctypes.c_float),
        ("fc2_input_scale", ctypes.c_float), ("routed_scaling_factor", ctypes.c_float),
        ("activation", ctypes.c_int), ("situ_beta", ctypes.c_float), ("situ_linear_beta", ctypes.c_float),
        ("w1_alpha_up", ctypes.c_void_p), ("per_token_scale", ctypes.c_void_p),
        ("fc1_bias", ctypes.c_void_p), ("fc2_bias", ctypes.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        sig = {
            "orc_e2m1_value": ([I], D), "orc_e4m3_value": ([I], D), "orc_e8m0_value": ([I], D),
            "orc_bf16_round": ([D], ctypes.c_uint16), "orc_e4m3_encode": ([F], I), "orc_e2m1_encode": ([F], I),
            "orc_bf16_round_array": ([P, I64, P], None), "orc_e4m3_encode_array": ([P, I64, P], None),
            "orc_e2m1_encode_array": ([P, I64, P], None),
            "orc_nvfp4_global_scale": ([F], F),
            "orc_nvfp4_quantize": ([P, I64, I64, I64, F, P, P], None),
            "orc_mx_quantize": ([P, I64, I64, I64, I, P, P], None),
            "orc_amax_bf16": ([P, I64], F),
            "orc_nvfp4_quantize_bf16": ([P, I64, I64, P, P], F),
            "orc_mx_quantize_bf16": ([P, I64, I64, I, P, P], None),
            "orc_route_slots": ([I64, I, I, I], I64),
            "orc_sort": ([P, I64, I, I, I, I, P, P, P, P, P, P, P], None),
            "orc_swiglu": ([F, F, F, F, F], D),
            "orc_geglu_tanh": ([F, F], D),
            "orc_situ": ([F, F, F, F], D),
            "orc_gemm1_route": ([P, I64, I, P, P, P, P], None),
            "orc_gemm2_route": ([P, I, P, P], None),
            "orc_finalize": ([P, P, P, I64, I, I, F, I, P, P], None),
            "orc_forward_tokens": ([P, P, I, I, P, P], None),
            "orc_forward_plan": ([P, I, P, P, P, P, P, P, P, P, P, P, I, P, P], None),
            "orc_fc2_input_scale": ([P], F),
            "orc_num_threads": ([], I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "arrays must be C-contiguous numpy arrays"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(code)


def bf16_round(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_round_array(_p(v), v.size, _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e2m1_encode_array(_p(v), v.size, _p(out))
    return out


def swiglu(g: float, u: float, alpha=1.0, beta=0.0, limit=float(np.finfo(np.float32).max)) -> float:
    return lib().orc_swiglu(g, u, alpha, beta, limit)


def geglu_tanh(g: float, u: float) -> float:
    """gelu_tanh(g) * u in fp64 (activation_type GegluTanh)"""
    return lib().orc_geglu_tanh(g, u)


def situ(g: float, u: float, beta: float, linear_beta: float = 0.0) -> float:
    """SiTU gate beta * tanh(g / beta) * sigmoid(g) times the up branch,
    clamped by linear_beta * tanh(u / linear_beta) when linear_beta > 0"""
    return lib().orc_situ(g, u, beta, linear_beta)


# ---------------------------------------------------------------- quantisers
def nvfp4_global_scale(amax: float) -> float:
    return lib().orc_nvfp4_global_scale(amax)


def nvfp4_quantize(v: np.ndarray, gscale: float):
    """fp32 [rows, cols] -> (packed codes uint8 [rows, cols/2], E4M3 scales uint8 [rows, cols/16])."""
    v = np.ascontiguousarray(v, np.float32)
    rows, cols = v.shape
    assert cols % 16 == 0
    q = np.zeros((rows, cols // 2), np.uint8)
    sf = np.zeros((rows, cols // 16), np.uint8)
    lib().orc_nvfp4_quantize(_p(v), rows, cols, cols, gscale, _p(q), _p(sf))
    return q, sf


def mx_quantize(v: np.ndarray, elem: int):
    """fp32 [rows, cols] -> (codes, E8M0 scales [rows, cols/32]); E4M3 one byte per element, E2M1 packed."""
    v = np.ascontiguousarray(v, np.float32)
    rows, cols = v.shape
    assert cols % 32 == 0
    q = np.zeros((rows, cols if elem == ELEM_E4M3 else cols // 2), np.uint8)
    sf = np.zeros((rows, cols // 32), np.uint8)
    lib().orc_mx_quantize(_p(v), rows, cols, cols, elem, _p(q), _p(sf))
    return q, sf


def amax_bf16(v: np.ndarray) -> float:
    v = np.ascontiguousarray(v, np.uint16)
    return lib().orc_amax_bf16(_p(v), v.size)


def nvfp4_quantize_bf16(v: np.ndarray):
    """bf16 bits [..., cols] quantised with a per-tensor global scale from its amax.
    Returns (codes [..., cols/2], scales [..., cols/16], global scale)."""
    v = np.ascontiguousarray(v, np.uint16)
    cols = v.shape[-1]
    rows = v.size // cols
    q = np.zeros(v.shape[:-1] + (cols // 2,), np.uint8)
    sf = np.zeros(v.shape[:-1] + (cols // 16,), np.uint8)
    gs = lib().orc_nvfp4_quantize_bf16(_p(v), rows, cols, _p(q), _p(sf))
    return q, sf, gs


def mx_quantize_bf16(v: np.ndarray, elem: int):
    v = np.ascontiguousarray(v, np.uint16)
    cols = v.shape[-1]
    rows = v.size // cols
    q = np.zeros(v.shape[:-1] + ((cols if elem == ELEM_E4M3 else cols // 2),), np.uint8)
    sf = np.zeros(v.shape[:-1] + (cols // 32,), np.uint8)
    lib().orc_mx_quantize_bf16(_p(v), rows, cols, elem, _p(q), _p(sf))
    return q, sf


# ---------------------------------------------------------------- routing plan
def route_slots(M: int, top_k: int, num_local_experts: int, tile: int) -> int:
    return lib().orc_route_slots(M, top_k, num_local_experts, tile)


@dataclass
class Plan:
    tile: int
    expanded_to_permuted: np.ndarray  # int32 [M*k]
    permuted_to_expanded: np.ndarray  # int32 [slots]
    tile_to_expert: np.ndarray        # int32 [slots/tile]
    tile_to_mn_limit: np.ndarray      # int32 [slots/tile]
    num_tiles: int
    expert_offsets: np.ndarray        # int32 [E_l+1]
    expert_counts: np.ndarray         # int32 [E_l]


def _plan_arrays(M, k, El, tile):
    slots = route_slots(M, k, El, tile)
    return (np.zeros(M * k, np.int32), np.zeros(slots, np.int32), np.zeros(slots // tile, np.int32),
            np.zeros(slots // tile, np.int32), np.zeros(1, np.int32), np.zeros(El + 1, np.int32),
            np.zeros(El, np.int32))


def sort(topk_ids: np.ndarray, num_local_experts: int, local_expert_offset: int, tile: int) -> Plan:
    ids = np.ascontiguousarray(topk_ids, np.int32)
    M, k = ids.shape
    arr = _plan_arrays(M, k, num_local_experts, tile)
    lib().orc_sort(_p(ids), M, k, num_local_experts, local_expert_offset, tile, *[_p(a) for a in arr])
    return Plan(tile, arr[0], arr[1], arr[2], arr[3], int(arr[4][0]), arr[5], arr[6])


# ---------------------------------------------------------------- forward
@dataclass
class Problem:
    """A quantised problem exactly as the forward pass receives it."""
    mode: int
    M: int
    H: int
    I: int
    top_k: int
    num_experts: int
    num_local_experts: int
    local_expert_offset: int
    x: np.ndarray                # bf16 bits [M,H] | packed [M,H/2] | E4M3 [M,H]
    x_sf: np.ndarray | None
    topk_ids: np.ndarray
    topk_weights: np.ndarray
    w1: np.ndarray
    w1_sf: np.ndarray
    w1_alpha: np.ndarray
    w2: np.ndarray
    w2_sf: np.ndarray
    w2_alpha: np.ndarray
    swiglu_alpha: float = 1.0
    swiglu_beta: float = 0.0
    swiglu_limit: float = float(np.finfo(np.float32).max)
    fc2_input_scale: float = 0.0
    routed_scaling_factor: float = 1.0
    x_row_stride: int = 0        # 0: contiguous
    activation: int = 0          # ACT_SWIGLU (SiTU when situ_beta > 0) | ACT_GEGLU_TANH
    situ_beta: float = 0.0
    situ_linear_beta: float = 0.0
    w1_alpha_up: np.ndarray | None = None      # fp32 [E_l]: the up half's own scale (None: w1_alpha)
    per_token_scale: np.ndarray | None = None  # fp32 [M], W4A4: GEMM1 input row scale
    fc1_bias: np.ndarray | None = None         # fp32 [E_l, 2I]: GEMM1 bias (gate rows, then up rows)
    fc2_bias: np.ndarray | None = None         # fp32 [E_l, H]: GEMM2 bias

    def struct(self) -> _Moe:
        s = _Moe()
        s.mode, s.M, s.H, s.I = self.mode, self.M, self.H, self.I
        s.top_k, s.num_experts, s.num_local_experts = self.top_k, self.num_experts, self.num_local_experts
        s.local_expert_offset = self.local_expert_offset
        for name in ("x", "x_sf", "topk_ids", "topk_weights", "w1", "w1_sf", "w1_alpha", "w2", "w2_sf", "w2_alpha",
                     "w1_alpha_up", "per_token_scale", "fc1_bias", "fc2_bias"):
            a = getattr(self, name)
            if a is not None:
                assert a.flags["C_CONTIGUOUS"], name
            setattr(s, name, None if a is None else a.ctypes.data)
        stride = self.x_row_stride or self.x.shape[-1]
        s.x_row_stride = stride
        s.swiglu_alpha, s.swiglu_beta, s.swiglu_limit = self.swiglu_alpha, self.swiglu_beta, self.swiglu_limit
        s.fc2_input_scale, s.routed_scaling_factor = self.fc2_input_scale, self.routed_scaling_factor
        s.activation, s.situ_beta, s.situ_linear_beta = self.activation, self.situ_beta, self.situ_linear_beta
        self._keep = s
        return s


def y1_shapes(mode: int, slots: int, I: int):
    if mode == W4A16:
        return (slots, I), np.uint16, None
    if mode == W4A4:
        return (slots, I // 2), np.uint8, (slots, I // 16)
    return (slots, I), np.uint8, (slots, I // 32)


def forward_plan(p: Problem, tile: int, accumulate: bool = False, out_prev: np.ndarray | None = None):
    """Plan-based oracle.  Returns (plan, y1, y1_sf, y2, out)."""
    arr = _plan_arrays(p.M, p.top_k, p.num_local_experts, tile)
    slots = arr[1].size
    s1, dt1, s1sf = y1_shapes(p.mode, slots, p.I)
    y1 = np.zeros(s1, dt1)
    y1_sf = None if s1sf is None else np.zeros(s1sf, np.uint8)
    y2 = np.zeros((slots, p.H), np.uint16)
    out = np.zeros((p.M, p.H), np.uint16)
    if accumulate:
        out_prev = np.ascontiguousarray(out_prev, np.uint16)
    st = p.struct()
    lib().orc_forward_plan(ctypes.byref(st), tile, *[_p(a) for a in arr], _p(y1), _p(y1_sf), _p(y2),
                           int(accumulate), _p(out_prev) if accumulate else None, _p(out))
    plan = Plan(tile, arr[0], arr[1], arr[2], arr[3], int(arr[4][0]), arr[5], arr[6])
    return plan, y1, y1_sf, y2, out


def forward_tokens(p: Problem, tokens, accumulate: bool = False, out_prev: np.ndarray | None = None) -> np.ndarray:
    """Per-token brute force (no plan): bf16 bits [len(tokens), H]."""
    tokens = np.ascontiguousarray(tokens, np.int32)
    out = np.zeros((tokens.size, p.H), np.uint16)
    if accumulate:
        out_prev = np.ascontiguousarray(out_prev, np.uint16)
        assert out_prev.shape == out.shape
    st = p.struct()
    lib().orc_forward_tokens(ctypes.byref(st), _p(tokens), tokens.size, int(accumulate),
                             _p(out_prev) if accumulate else None, _p(out))
    return out


def gemm1_route(p: Problem, t: int, le: int):
    """(y1 bf16 [I], y1 codes, y1 scales, decoded GEMM2 input fp64 [I]) for one route."""
    y1 = np.zeros(p.I, np.uint16)
    s1, dt1, s1sf = y1_shapes(p.mode, 1, p.I)
    q = np.zeros(s1[1], np.uint8) if p.mode != W4A16 else None
    sf = np.zeros(s1sf[1], np.uint8) if s1sf else None
    a2 = np.zeros(p.I, np.float64)
    st = p.struct()
    lib().orc_gemm1_route(ctypes.byref(st), t, le, _p(y1), _p(q), _p(sf), _p(a2))
    return y1, q, sf, a2


def gemm2_route(p: Problem, le: int, a2: np.ndarray) -> np.ndarray:
    a2 = np.ascontiguousarray(a2, np.float64)
    y2 = np.zeros(p.H, np.uint16)
    st = p.struct()
    lib().orc_gemm2_route(ctypes.byref(st), le, _p(a2), _p(y2))
    return y2


def finalize(y2: np.ndarray, e2p: np.ndarray, topk_weights: np.ndarray, H: int, rsf: float = 1.0,
             accumulate: bool = False, out_prev: np.ndarray | None = None) -> np.ndarray:
    y2 = np.ascontiguousarray(y2, np.uint16)
    e2p = np.ascontiguousarray(e2p, np.int32)
    w = np.ascontiguousarray(topk_weights, np.float32)
    M, k = w.shape
    out = np.zeros((M, H), np.uint16)
    if accumulate:
        out_prev = np.ascontiguousarray(out_prev, np.uint16)
    lib().orc_finalize(_p(y2), _p(e2p), _p(w), M, k, H, rsf, int(accumulate),
                       _p(out_prev) if accumulate else None, _p(out))
    return out


def fc2_input_scale(p: Problem) -> float:
    st = p.struct()
    return lib().orc_fc2_input_scale(ctypes.byref(st))


def num_threads() -> int:
    return lib().orc_num_threads()


# ---------------------------------------------------------------- problem preparation
def quantize_problem(raw, calibrate: bool = True) -> Problem:
    """Quantise a synth.RawInputs workload the way the recipe states:
    weights per expert to NVFP4 (global scale amax/(6*448), E4M3 block-16
    scales) or MXFP4 (E8M0 block-32); x to NVFP4 (per-tensor scale) for W4A4
    or MXFP8 for the MX mode.  W4A4 folds the activation scales into the
    per-expert alphas and calibrates fc2_input_scale with a first pass."""
    wl = raw.wl
    E, H, I = wl.num_local_experts, wl.H, wl.I
    if wl.mode == MXFP8_MXFP4:
        w1, w1_sf = mx_quantize_bf16(raw.w1, ELEM_E2M1)
        w2, w2_sf = mx_quantize_bf16(raw.w2, ELEM_E2M1)
        a1 = np.ones(E, np.float32)
        a2 = np.ones(E, np.float32)
    else:
        w1 = np.zeros((E, raw.w1.shape[1], H // 2), np.uint8)
        w1_sf = np.zeros((E, raw.w1.shape[1], H // 16), np.uint8)
        w2 = np.zeros((E, H, I // 2), np.uint8)
        w2_sf = np.zeros((E, H, I // 16), np.uint8)
        a1 = np.zeros(E, np.float32)
        a2 = np.zeros(E, np.float32)
        for e in range(E):
            w1[e], w1_sf[e], a1[e] = nvfp4_quantize_bf16(raw.w1[e])
            w2[e], w2_sf[e], a2[e] = nvfp4_quantize_bf16(raw.w2[e])
    x_sf = None
    if wl.mode == W4A16:
        x = raw.x
    elif wl.mode == W4A4:
        x, x_sf, ax = nvfp4_quantize_bf16(raw.x)
        a1 = (a1 * np.float32(ax)).astype(np.float32)
    else:
        x, x_sf = mx_quantize_bf16(raw.x, ELEM_E4M3)
    p = Problem(wl.mode, wl.M, H, I, wl.top_k, wl.num_experts, E, wl.local_expert_offset,
                np.ascontiguousarray(x), x_sf, raw.topk_ids, raw.topk_weights, w1, w1_sf, a1, w2, w2_sf, a2,
                swiglu_alpha=wl.swiglu_alpha, swiglu_beta=wl.swiglu_beta, swiglu_limit=wl.swiglu_limit,
                activation=wl.activation, situ_beta=wl.situ_beta, situ_linear_beta=wl.situ_linear_beta)
    if wl.mode == W4A4:
        p.extra_w2_alpha_raw = a2.copy()
        if calibrate:
            fs = fc2_input_scale(p)
            set_fc2_input_scale(p, fs)
    return p


def set_fc2_input_scale(p: Problem, fs: float):
    """W4A4: the FC1-output global scale and its fold into w2_alpha."""
    p.fc2_input_scale = float(np.float32(fs))
    p.w2_alpha = (p.extra_w2_alpha_raw * np.float32(fs)).astype(np.float32)
