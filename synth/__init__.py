"""Seeded synthetic inputs for the fused MoE forward (shared by the oracle's
tests and the GPU benchmark; holds none of the method's arithmetic).

The C core (``synth.c``) draws SplitMix64 numbers counter-style and turns
them into normals (Box-Muller); this module wraps it with numpy and defines
the workloads: their shapes, distributions and seeds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# stream ids, one per tensor
STREAM_X, STREAM_LOGITS, STREAM_BIAS, STREAM_W1, STREAM_W2 = 1, 2, 3, 4, 5


def build(force: bool = True) -> str:
    """Compile libsynth.so next to its source (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_double, P]
        L.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_double, P]
        L.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, P]
        L.synth_router.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P]
        L.synth_sample_tokens.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, P]
        L.synth_mix64.argtypes = [ctypes.c_uint64]
        L.synth_mix64.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_f32(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(seed, stream, out.size, mean, std, _p(out))
    return out


def normal_bf16(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(mean, std) draws."""
    out = np.empty(shape, np.uint16)
    lib().synth_normal_bf16(seed, stream, out.size, mean, std, _p(out))
    return out


def u64(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_u64(seed, stream, n, _p(out))
    return out


def router(logits: np.ndarray, bias: np.ndarray | None, k: int):
    """top-k expert ids (int32 [M,k]) and renormalised weights (fp32 [M,k])."""
    logits = np.ascontiguousarray(logits, np.float32)
    M, E = logits.shape
    assert k <= 64 and k <= E
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().synth_router(_p(logits), None if b is None else _p(b), M, E, k, _p(ids), _p(w))
    return ids, w


def sample_tokens(seed: int, M: int, n: int) -> np.ndarray:
    n = min(n, M)
    out = np.empty(n, np.int32)
    lib().synth_sample_tokens(seed, M, n, _p(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
W4A16, W4A4, MXFP8_MXFP4 = 0, 1, 2
MODE_NAMES = {W4A16: "w4a16", W4A4: "w4a4", MXFP8_MXFP4: "mxfp8_mxfp4"}


@dataclass(frozen=True)
class Workload:
    name: str
    mode: int
    M: int
    H: int
    I: int
    num_experts: int
    num_local_experts: int
    top_k: int
    seed: int
    local_expert_offset: int = 0
    router_bias_std: float = 0.0      # per-expert bias N(0, std) added to the logits
    swiglu_alpha: float = 1.0
    swiglu_beta: float = 0.0
    swiglu_limit: float = float(np.finfo(np.float32).max)
    activation: int = 0               # 0 SwiGLU (SiTU when situ_beta > 0), 1 GeGLU-tanh, 2 ReLU^2
    situ_beta: float = 0.0
    situ_linear_beta: float = 0.0
    x_std: float = 1.0
    w_std: float = 0.02
    sample_tokens: int = 0            # >0: parity on this many sampled tokens
    notes: str = ""

    @property
    def routes(self) -> int:
        return self.M * self.top_k


WORKLOADS = {
    "w4a16_tiny": Workload("w4a16_tiny", W4A16, M=16, H=256, I=512, num_experts=8,
                           num_local_experts=8, top_k=2, seed=0),
    "w4a16_decode": Workload("w4a16_decode", W4A16, M=8, H=6144, I=2048, num_experts=256,
                             num_local_experts=32, top_k=8, seed=1),
    "w4a16_prefill": Workload("w4a16_prefill", W4A16, M=4096, H=6144, I=2048, num_experts=256,
                              num_local_experts=32, top_k=8, seed=2, router_bias_std=0.5,
                              swiglu_limit=7.0),
    "w4a4_nvfp4": Workload("w4a4_nvfp4", W4A4, M=512, H=4096, I=1536, num_experts=128,
                           num_local_experts=128, top_k=8, seed=3),
    "mxfp8_mxfp4_large": Workload("mxfp8_mxfp4_large", MXFP8_MXFP4, M=65536, H=6144, I=2048,
                                  num_experts=256, num_local_experts=32, top_k=8, seed=4,
                                  sample_tokens=1024),
}


@dataclass
class RawInputs:
    """Unquantised draws of one workload: bf16 bit patterns and the routing."""
    wl: Workload
    x: np.ndarray            # bf16 [M, H]
    topk_ids: np.ndarray     # int32 [M, k]
    topk_weights: np.ndarray # fp32 [M, k]
    w1: np.ndarray | None = None  # bf16 [E_l, 2I, H]   (rows [0,I) gate, [I,2I) up)
    w2: np.ndarray | None = None  # bf16 [E_l, H, I]
    extra: dict = field(default_factory=dict)


def make_routing(wl: Workload):
    logits = normal_f32(wl.seed, STREAM_LOGITS, (wl.M, wl.num_experts))
    bias = None
    if wl.router_bias_std > 0:
        bias = normal_f32(wl.seed, STREAM_BIAS, (wl.num_experts,), 0.0, wl.router_bias_std)
    return router(logits, bias, wl.top_k)


def make_raw(wl: Workload, weights: bool = True) -> RawInputs:
    x = normal_bf16(wl.seed, STREAM_X, (wl.M, wl.H), 0.0, wl.x_std)
    ids, w = make_routing(wl)
    raw = RawInputs(wl, x, ids, w)
    if weights:
        E = wl.num_local_experts
        rows = wl.I if wl.activation == 2 else 2 * wl.I   # ReLU^2 is non-gated: I rows
        raw.w1 = normal_bf16(wl.seed, STREAM_W1, (E, rows, wl.H), 0.0, wl.w_std)
        raw.w2 = normal_bf16(wl.seed, STREAM_W2, (E, wl.H, wl.I), 0.0, wl.w_std)
    return raw


def small_workload(mode: int, M: int, H: int, I: int, E: int, El: int, k: int, seed: int,
                   offset: int = 0, **kw) -> Workload:
    """An ad-hoc small workload for parity cases (same recipe, other shapes)."""
    return Workload(f"small_{MODE_NAMES[mode]}_{M}x{H}x{I}_e{E}_{El}_k{k}_s{seed}", mode, M=M, H=H, I=I,
                    num_experts=E, num_local_experts=El, top_k=k, seed=seed,
                    local_expert_offset=offset, **kw)
