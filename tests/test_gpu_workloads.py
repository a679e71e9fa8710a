"""The five workloads at full size on the GPU against the oracle: the plan
bit for bit, and the output on every token (small M) or on sampled tokens
the oracle evaluates one by one (large M), in the launch configuration the
benchmark times (default tile, deterministic finalize), plus the atomic
finalize."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _tokens(wl):
    if wl.sample_tokens:
        return synth.sample_tokens(wl.seed, wl.M, wl.sample_tokens)
    return np.arange(wl.M, dtype=np.int32)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload(name):
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import DeviceProblem, check_close, host, say
    wl = synth.WORKLOADS[name]
    say(f"workload {name}: generating and quantising on the host")
    p = oracle.quantize_problem(synth.make_raw(wl))
    d = DeviceProblem(p)
    tile = moe.default_tile(p.M, p.top_k, p.num_local_experts, p.mode)
    say(f"workload {name}: forward, tile {tile}")
    out = d.forward()
    torch.cuda.synchronize()
    plan = moe.moe_sort(d.ids, p.num_experts, p.num_local_experts, p.local_expert_offset, tile)
    torch.cuda.synchronize()
    ref_plan = oracle.sort(p.topk_ids, p.num_local_experts, p.local_expert_offset, tile)
    assert np.array_equal(host(plan.permuted_to_expanded), ref_plan.permuted_to_expanded)
    assert np.array_equal(host(plan.expanded_to_permuted), ref_plan.expanded_to_permuted)
    toks = _tokens(wl)
    say(f"workload {name}: oracle on {toks.size} tokens")
    want = oracle.forward_tokens(p, toks)
    got = host(out, np.uint16)[toks]
    check_close(got, want, p.mode, f"{name} deterministic")
    out_a = torch.zeros_like(out)
    d.forward(out=out_a, finalize_mode=moe.FINALIZE_ATOMIC)
    torch.cuda.synchronize()
    check_close(host(out_a, np.uint16)[toks], want, p.mode, f"{name} atomic")
