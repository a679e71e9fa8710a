"""The five workloads at full size on the GPU against the oracle: the plan
bit for bit, and the output on every token (small M) or on sampled tokens
the oracle evaluates one by one (large M), in the launch configuration the
benchmark times (default tile, deterministic finalize), plus the atomic
finalize.

Requantising modes (W4A4, MXFP8 x MXFP4) are also checked in stages, since
the y1 code is an integer decided from a bf16 value that the GPU (fp32
accumulation) and the oracle (fp64) may round to neighbouring values:
  * GEMM1: the GPU's y1 values agree with the oracle's almost everywhere
    (>= 99.5% of values, >= 95% of whole blocks: scale code and every
    element code), and every block that differs is still a valid
    quantisation: each decoded value within one code step;
  * GEMM2 + finalize: the oracle run from the GPU's own y1 codes meets the
    full bar against the GPU output."""
import numpy as np
import pytest

import oracle
import reference_np as ref
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
    requant = p.mode != oracle.W4A16
    check_close(got, want, p.mode, f"{name} deterministic", max_bar=not requant)
    out_a = torch.zeros_like(out)
    d.forward(out=out_a, finalize_mode=moe.FINALIZE_ATOMIC)
    torch.cuda.synchronize()
    check_close(host(out_a, np.uint16)[toks], want, p.mode, f"{name} atomic", max_bar=not requant)
    if requant:
        staged_requant_check(p, d, plan, toks, got, name)


def _decode_y1(mode, q, sf):
    """decoded y1 (the GEMM2 input) from codes and block scales"""
    if mode == oracle.W4A4:
        return ref.e2m1_vals(ref.unpack(q)) * np.repeat(ref.e4m3_vals(sf), 16, axis=-1)
    return ref.e4m3_vals(q) * np.repeat(ref.e8m0_vals(sf), 32, axis=-1)


def _code_step(mode, v, sf):
    """the spacing of neighbouring codes around |v| under block scale sf"""
    if mode == oracle.W4A4:
        scale = np.repeat(ref.e4m3_vals(sf), 16, axis=-1)
        return 2.0 * scale  # E2M1's widest gap (4 -> 6)
    scale = np.repeat(ref.e8m0_vals(sf), 32, axis=-1)
    return np.maximum(np.abs(v) / 8.0, 2.0 ** -9 * scale)  # E4M3: 3 mantissa bits; subnormal step


def staged_requant_check(p, d, plan, toks, got, name):
    import torch

    import mixture_experts_forward_moe_amd as moe
    from gpu_util import check_close, host, say
    slots = plan.route_slots
    s1, dt1, s1sf = oracle.y1_shapes(p.mode, slots, p.I)
    y1 = torch.zeros(s1, dtype=torch.uint8, device="cuda")
    y1_sf = torch.zeros(s1sf, dtype=torch.uint8, device="cuda")
    moe.moe_grouped_gemm1_swiglu(p.mode, d.x, d.x_sf, plan, d.w1, d.w1_sf, d.w1_alpha, p.H, p.I, y1, y1_sf,
                                 p.swiglu_alpha, p.swiglu_beta, p.swiglu_limit, d.fc2)
    torch.cuda.synchronize()
    e2p = host(plan.expanded_to_permuted).reshape(p.M, p.top_k)
    blk = 16 if p.mode == oracle.W4A4 else 32
    k = p.top_k
    y2 = np.zeros((toks.size * k, p.H), np.uint16)
    e2p_c = np.full((toks.size, k), -1, np.int32)
    same = total = same_el = total_el = 0
    say(f"{name}: staged check on {toks.size} tokens")
    for i, t in enumerate(toks):
        for j in range(k):
            s = int(e2p[t, j])
            if s < 0:
                continue
            le = int(p.topk_ids[t, j]) - p.local_expert_offset
            _, q_o, sf_o, a2_o = oracle.gemm1_route(p, int(t), le)
            q_g = host(y1[s])
            sf_g = host(y1_sf[s])
            a2_g = _decode_y1(p.mode, q_g, sf_g)
            # block agreement: the scale code and every element code
            codes_g = q_g.reshape(-1, blk // 2 if p.mode == oracle.W4A4 else blk)
            codes_o = q_o.reshape(codes_g.shape)
            eq = (sf_g == sf_o) & np.all(codes_g == codes_o, axis=1)
            same += int(eq.sum())
            total += eq.size
            same_el += int(np.sum(a2_g == a2_o))
            total_el += a2_g.size
            # a differing block is still a valid quantisation: one code step
            step = np.maximum(_code_step(p.mode, a2_g, sf_g), _code_step(p.mode, a2_o, sf_o))
            assert np.all(np.abs(a2_g - a2_o) <= step * (1 + 1e-12)), (name, int(t), j)
            y2[i * k + j] = oracle.gemm2_route(p, le, a2_g)
            e2p_c[i, j] = i * k + j
    agree = same / max(total, 1)
    agree_el = same_el / max(total_el, 1)
    say(f"{name}: y1 identical to the oracle's: {agree_el:.5f} of {total_el} values, {agree:.5f} of {total} blocks")
    # a value takes the neighbouring code only when its bf16 y1 moved by an
    # ulp across a code boundary (about 1 in 16 of a code interval for E4M3
    # from bf16); a block differs when any of its 16 or 32 values does
    assert agree_el >= 0.995, agree_el
    assert agree >= 0.95, agree
    staged = oracle.finalize(y2, e2p_c, p.topk_weights[toks], p.H, p.routed_scaling_factor)
    check_close(got, staged, p.mode, f"{name} from the GPU's own y1")
