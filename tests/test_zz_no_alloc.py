"""moe_forward_noalloc through the C ABI against moe_forward on the same
inputs: two calls in a row on the library's scratch array, the second with a
smaller input, each bit for bit equal to moe_forward's deterministic result
(the same kernels on the same plan) and within the bar against the oracle,
and the atomic finalize within the bar.  (The refusal of a pass larger than
the array is a host check, covered without a GPU.)"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _problem(name):
    if name in synth.WORKLOADS:
        return oracle.quantize_problem(synth.make_raw(synth.WORKLOADS[name]))
    # a tiled-path W4A4 problem (tile 32) that fits the scratch array
    wl = synth.small_workload(oracle.W4A4, 48, 1024, 512, 16, 8, 4, 71, offset=4)
    return oracle.quantize_problem(synth.make_raw(wl))


def _noalloc(d, out, **kw):
    import mixture_experts_forward_moe_amd as moe
    p = d.p
    return moe.moe_forward_noalloc(d.x, d.x_sf, d.ids, d.w, d.w1, d.w1_sf, d.w1_alpha, d.w2, d.w2_sf, d.w2_alpha,
                                   p.num_experts, p.top_k, p.num_local_experts, p.local_expert_offset, p.mode, out,
                                   p.H, p.I, swiglu_alpha=p.swiglu_alpha, swiglu_beta=p.swiglu_beta,
                                   swiglu_limit=p.swiglu_limit, fc2_input_scale=d.fc2, **kw)


def test_noalloc_matches_forward():
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import DeviceProblem, check_close, host, say
    # two calls in a row, the second smaller: the decode workload (two-launch
    # path), then the tiny workload; then a tiled-path W4A4 problem
    for name in ("w4a16_decode", "w4a16_tiny", "w4a4_small"):
        say(f"noalloc: {name}")
        p = _problem(name)
        d = DeviceProblem(p)
        want = d.forward()
        got = torch.full_like(want, 0x1234)
        _noalloc(d, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), name
        check_close(host(got, np.uint16), oracle.forward_tokens(p, np.arange(p.M)), p.mode, f"noalloc {name}")
        got_a = torch.zeros_like(want)
        _noalloc(d, got_a, finalize_mode=moe.FINALIZE_ATOMIC)
        torch.cuda.synchronize()
        check_close(host(got_a, np.uint16), host(want, np.uint16), p.mode, f"noalloc {name} atomic")
