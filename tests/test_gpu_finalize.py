"""moe_finalize on the GPU against the oracle, bit for bit, given the same
y2: overwrite and accumulate, a routed scaling factor, non-local routes."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,k,El,E,H,tile,acc,rsf", [
    (16, 2, 8, 8, 256, 16, False, 1.0),
    (8, 8, 32, 256, 6144, 16, False, 1.0),
    (300, 8, 32, 256, 1024, 64, True, 0.75),
    (1000, 4, 16, 16, 2048, 32, False, 2.5),
])
def test_finalize_bit_exact(M, k, El, E, H, tile, acc, rsf):
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import dev, host, say
    say(f"finalize M={M} k={k} El={El} H={H} acc={acc} rsf={rsf}")
    rng = np.random.default_rng(M + H)
    ids = rng.integers(0, E, (M, k)).astype(np.int32)
    w = rng.random((M, k)).astype(np.float32)
    plan = moe.moe_sort(dev(ids), E, El, 0, tile)
    ref_plan = oracle.sort(ids, El, 0, tile)
    y2 = synth.normal_bf16(7, 1, (plan.route_slots, H))
    prev = synth.normal_bf16(7, 2, (M, H))
    out = dev(prev.copy())
    moe.moe_finalize(dev(y2), plan, dev(w), H, out, routed_scaling_factor=rsf, accumulate=acc)
    torch.cuda.synchronize()
    ref = oracle.finalize(y2, ref_plan.expanded_to_permuted, w, H, rsf=rsf, accumulate=acc, out_prev=prev)
    assert np.array_equal(host(out, np.uint16), ref)
