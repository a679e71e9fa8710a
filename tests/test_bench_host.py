"""Host-side checks of the benchmark's work accounting (no GPU): the
algorithmic bytes and flops its roofline fractions are computed from."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_decode_bytes_closed_form():
    """W4A16 decode shape (H 6144, I 2048): an active expert's NVFP4 W1 + W2
    are 21,233,664 bytes (codes at 4 bits, an E4M3 scale per 16); per route
    its x row, y1 written and read, and y2 written and read
    (deterministic) or the row added into out (atomic); the output once."""
    wl = synth.WORKLOADS["w4a16_decode"]
    H, I, M, k = wl.H, wl.I, wl.M, wl.top_k
    per_expert = 3 * H * I // 2 + 3 * H * I // 16
    assert per_expert == 21_233_664
    routes, active = 7, 7
    det = bench.w4a16_bytes(wl, routes, active)
    ato = bench.w4a16_bytes(wl, routes, active, atomic=True)
    io = M * k * 8 + M * H * 2
    assert det["weights"] == active * per_expert == ato["weights"]
    assert det["forward"] == active * per_expert + routes * (2 * H + 4 * I + 4 * H) + io
    assert ato["forward"] == active * per_expert + routes * (2 * H + 4 * I + 2 * H) + io
    # GEMM1 also clears out in the atomic mode
    assert ato["gemm1"] - det["gemm1"] == M * H * 2
    assert det["gemm1"] + det["gemm2"] == det["weights"] + routes * (2 * H + 2 * I + 2 * I + 2 * H)


def test_relu2_has_half_the_w1_rows():
    """The non-gated ReLU^2 FC1 has I rows, not 2I."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["w4a16_decode"], activation=2)
    b = bench.w4a16_bytes(wl, 1, 1)
    assert b["w1_per_expert"] == wl.I * wl.H // 2 + wl.I * wl.H // 16
    assert b["w2_per_expert"] == wl.H * wl.I // 2 + wl.H * wl.I // 16


@pytest.mark.parametrize("name", ["w4a16_prefill", "mxfp8_mxfp4_large"])
def test_flops_per_route(name):
    """6 H I flops per route: 4 H I for the gated GEMM1 (2I rows), 2 H I for GEMM2."""
    wl = synth.WORKLOADS[name]
    assert bench.flops(wl, 1000) == 6.0 * wl.H * wl.I * 1000


def test_weight_bytes_by_block_size():
    """NVFP4 carries a scale byte per 16 codes, MXFP4 per 32."""
    nv = synth.WORKLOADS["w4a16_prefill"]
    mx = synth.WORKLOADS["mxfp8_mxfp4_large"]
    assert bench.weight_bytes(nv, 1) == 3 * nv.H * nv.I // 2 + 3 * nv.H * nv.I // 16
    assert bench.weight_bytes(mx, 1) == 3 * mx.H * mx.I // 2 + 3 * mx.H * mx.I // 32
