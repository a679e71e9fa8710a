"""The library's NVFP4 / MX input quantisers against the oracle's, bit for bit."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batches,rows,cols,std", [(1, 64, 256, 1.0), (4, 96, 512, 0.02), (2, 8, 6144, 3.0)])
def test_nvfp4(batches, rows, cols, std):
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import dev, host, say
    say(f"quantize nvfp4 {batches}x{rows}x{cols}")
    x = synth.normal_bf16(3, 1, (batches, rows, cols), 0.0, std)
    gs = torch.zeros(batches, dtype=torch.float32, device="cuda")
    q = torch.zeros((batches, rows, cols // 2), dtype=torch.uint8, device="cuda")
    sf = torch.zeros((batches, rows, cols // 16), dtype=torch.uint8, device="cuda")
    xd = dev(x)
    moe.moe_nvfp4_global_scale(xd, batches, gs)
    moe.moe_quantize_nvfp4(xd, batches, rows, cols, gs, q, sf)
    torch.cuda.synchronize()
    for b in range(batches):
        rq, rs, rg = oracle.nvfp4_quantize_bf16(x[b])
        assert host(gs)[b] == np.float32(rg)
        assert np.array_equal(host(sf)[b], rs)
        assert np.array_equal(host(q)[b], rq)


@pytest.mark.parametrize("elem", [0, 1])
@pytest.mark.parametrize("rows,cols,std", [(64, 256, 1.0), (33, 6144, 0.02), (5, 2048, 1e-30)])
def test_mx(elem, rows, cols, std):
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import dev, host, say
    say(f"quantize mx elem={elem} {rows}x{cols}")
    x = synth.normal_bf16(4, 1, (rows, cols), 0.0, std)
    q = torch.zeros((rows, cols if elem == 0 else cols // 2), dtype=torch.uint8, device="cuda")
    sf = torch.zeros((rows, cols // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mx(dev(x), rows, cols, elem, q, sf)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize_bf16(x, elem)
    assert np.array_equal(host(sf), rs)
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("case", ["w4a4_nvfp4", "w4a4_small", "w4a4_relu2_scaled"])
def test_fc2_input_scale_calibration(case):
    """moe_fc2_input_scale (GEMM1 on the device with a max over |y1|) against
    the oracle's calibration pass: the same max over every local route of
    the bf16 FC1 output, divided by 6 * 448.  The GPU's y1 equals the
    oracle's on (almost) every value, so the scales agree to within one bf16
    step of the largest y1 (bit for bit when its value agrees)."""
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import DeviceProblem, say
    say(f"fc2_input_scale calibration {case}")
    if case == "w4a4_nvfp4":
        p = oracle.quantize_problem(synth.make_raw(synth.WORKLOADS[case]))
    else:
        act = oracle.ACT_RELU2 if "relu2" in case else oracle.ACT_SWIGLU
        wl = synth.small_workload(oracle.W4A4, 70, 384, 320, 16, 6, 3, 91, offset=3, activation=act)
        p = oracle.quantize_problem(synth.make_raw(wl))
        if "scaled" in case:
            rng = np.random.default_rng(92)
            p.per_token_scale = rng.uniform(0.25, 4.0, p.M).astype(np.float32)
            p.fc1_bias = rng.normal(0.0, 0.05, (p.num_local_experts, p.I)).astype(np.float32)
    want = oracle.fc2_input_scale(p)
    d = DeviceProblem(p)
    tile = moe.default_tile(p.M, p.top_k, p.num_experts, p.num_local_experts, p.mode)
    plan = moe.moe_sort(d.ids, p.num_experts, p.num_local_experts, p.local_expert_offset, tile)
    got = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_fc2_input_scale(d.x, d.x_sf, plan, d.w1, d.w1_sf, d.w1_alpha, p.H, p.I, got, activation=p.activation,
                            per_token_scale=d.pts, fc1_bias=d.fc1_bias)
    torch.cuda.synchronize()
    g = float(got.cpu()[0])
    say(f"{case}: fc2_input_scale gpu {g:.9g} oracle {want:.9g}")
    assert abs(g - want) <= want * 2.0 ** -7, (g, want)
