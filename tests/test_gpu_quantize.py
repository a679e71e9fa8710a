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
