"""Pins of the oracle's forward pass (GEMM1 + SwiGLU + requantisation, GEMM2,
finalize) against an independent numpy/torch statement built from library
routines, closed forms of the SwiGLU, hand-computed finalize values and the
invariants the pages state (accumulate=False equals accumulating onto
zeros; per-token and plan-based evaluation agree)."""
import math

import numpy as np
import pytest

import oracle
import reference_np as ref
import synth

FLT_MAX = float(np.finfo(np.float32).max)


def _problem(mode, M, H, I, E, El, k, seed, offset=0, **kw):
    wl = synth.small_workload(mode, M, H, I, E, El, k, seed, offset, **kw)
    return oracle.quantize_problem(synth.make_raw(wl))


def _close_bf16(a_bits, b_bits, min_exact=0.99, rel_l2=1e-3):
    a = synth.bf16_to_f32(a_bits).astype(np.float64)
    b = synth.bf16_to_f32(b_bits).astype(np.float64)
    exact = np.mean(a_bits == b_bits)
    err = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
    assert exact >= min_exact and err <= rel_l2, (exact, err)


SMALL = [
    (oracle.W4A16, dict(M=12, H=128, I=64, E=8, El=8, k=2, seed=21)),
    (oracle.W4A16, dict(M=10, H=64, I=96, E=16, El=5, k=4, seed=22, offset=6, swiglu_limit=0.02,
                        swiglu_alpha=1.702, swiglu_beta=1.0)),
    (oracle.W4A4, dict(M=12, H=128, I=64, E=8, El=8, k=2, seed=23)),
    (oracle.W4A4, dict(M=9, H=64, I=128, E=12, El=6, k=3, seed=24, offset=3)),
    (oracle.MXFP8_MXFP4, dict(M=12, H=128, I=64, E=8, El=8, k=2, seed=25)),
    (oracle.MXFP8_MXFP4, dict(M=9, H=96, I=128, E=12, El=4, k=3, seed=26, offset=8)),
    # the other gated FC1 activations: GeGLU-tanh, SiTU (with and without the up-branch clamp)
    (oracle.W4A16, dict(M=10, H=64, I=96, E=8, El=8, k=2, seed=27, activation=oracle.ACT_GEGLU_TANH)),
    (oracle.W4A16, dict(M=10, H=64, I=64, E=8, El=6, k=3, seed=28, offset=1, situ_beta=0.1,
                        situ_linear_beta=0.08)),
    (oracle.W4A4, dict(M=9, H=64, I=64, E=8, El=8, k=2, seed=29, situ_beta=0.1)),
    (oracle.MXFP8_MXFP4, dict(M=9, H=96, I=64, E=8, El=8, k=2, seed=30, activation=oracle.ACT_GEGLU_TANH)),
    # the non-gated ReLU^2 (W1 has I rows)
    (oracle.W4A16, dict(M=10, H=64, I=64, E=8, El=6, k=3, seed=31, offset=2, activation=oracle.ACT_RELU2)),
    (oracle.W4A4, dict(M=9, H=64, I=64, E=8, El=8, k=2, seed=36, activation=oracle.ACT_RELU2)),
    (oracle.MXFP8_MXFP4, dict(M=9, H=96, I=64, E=8, El=8, k=2, seed=37, activation=oracle.ACT_RELU2)),
]


@pytest.mark.parametrize("mode,kw", SMALL)
def test_oracle_matches_library_reference(mode, kw):
    p = _problem(mode, **kw)
    tokens = np.arange(p.M)
    got = oracle.forward_tokens(p, tokens)
    want = ref.forward_tokens(p, tokens)
    _close_bf16(got, want)


def test_tiny_workload_matches_library_reference():
    p = oracle.quantize_problem(synth.make_raw(synth.WORKLOADS["w4a16_tiny"]))
    tokens = np.arange(p.M)
    _close_bf16(oracle.forward_tokens(p, tokens), ref.forward_tokens(p, tokens))


@pytest.mark.parametrize("mode,kw", SMALL)
def test_plan_based_equals_per_token_bit_for_bit(mode, kw):
    p = _problem(mode, **kw)
    for tile in (1, 4, 16):
        plan, y1, y1_sf, y2, out = oracle.forward_plan(p, tile)
        assert np.array_equal(out, oracle.forward_tokens(p, np.arange(p.M)))


def test_accumulate_false_equals_accumulating_onto_zeros():
    p = _problem(oracle.W4A16, M=8, H=64, I=32, E=4, El=4, k=2, seed=31)
    _, _, _, y2, out = oracle.forward_plan(p, 8)
    plan = oracle.sort(p.topk_ids, 4, 0, 8)
    zeros = np.zeros_like(out)
    a = oracle.finalize(y2, plan.expanded_to_permuted, p.topk_weights, p.H, accumulate=False)
    b = oracle.finalize(y2, plan.expanded_to_permuted, p.topk_weights, p.H, accumulate=True, out_prev=zeros)
    assert np.array_equal(a, b) and np.array_equal(a, out)
    # accumulating onto a previous output adds to it
    prev = synth.normal_bf16(5, 9, out.shape)
    c = oracle.finalize(y2, plan.expanded_to_permuted, p.topk_weights, p.H, accumulate=True, out_prev=prev)
    d = oracle.forward_tokens(p, np.arange(p.M), accumulate=True, out_prev=prev)
    assert np.array_equal(c, d)


def test_finalize_hand_values():
    # two tokens, top_k 2, H 3; token 1's second route is not local
    y2 = np.array([[1.0, -2.0, 0.5], [4.0, 8.0, -1.0], [0.25, 0.0, 3.0]], np.float32)
    y2b = (y2.view(np.uint32) >> 16).astype(np.uint16)
    e2p = np.array([0, 1, 2, -1], np.int32)
    w = np.array([[0.5, 0.25], [2.0, 7.0]], np.float32)
    out = oracle.finalize(y2b, e2p, w, 3, rsf=1.0)
    want = np.array([[0.5 + 1.0, -1.0 + 2.0, 0.25 - 0.25], [0.5, 0.0, 6.0]], np.float32)
    assert np.array_equal(synth.bf16_to_f32(out), want)
    out2 = oracle.finalize(y2b, e2p, w, 3, rsf=0.5)
    assert np.array_equal(synth.bf16_to_f32(out2), want * 0.5)
    # k = 1 and weight 1: the output is y2 itself
    out3 = oracle.finalize(y2b, np.array([2, 0], np.int32), np.ones((2, 1), np.float32), 3)
    assert np.array_equal(out3, y2b[[2, 0]])


def test_swiglu_closed_forms():
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert oracle.swiglu(40.0, 3.0) == pytest.approx(120.0, rel=1e-15)
    assert abs(oracle.swiglu(-60.0, 3.0)) < 1e-20
    assert oracle.swiglu(2.0, 1.0) == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    # limit clamps g from above and u on both sides; alpha scales the sigmoid argument; beta shifts u
    lim = 7.0
    assert oracle.swiglu(9.0, 1.0, 1.0, 0.0, lim) == pytest.approx(7.0 / (1 + math.exp(-7.0)), rel=1e-15)
    assert oracle.swiglu(1.0, 9.0, 1.0, 0.0, lim) == pytest.approx(7.0 / (1 + math.exp(-1.0)), rel=1e-15)
    assert oracle.swiglu(1.0, -9.0, 1.0, 0.0, lim) == pytest.approx(-7.0 / (1 + math.exp(-1.0)), rel=1e-15)
    assert oracle.swiglu(-9.0, 1.0, 1.0, 0.0, lim) == pytest.approx(-9.0 / (1 + math.exp(9.0)), rel=1e-15)
    a32 = float(np.float32(1.702))   # the parameters are fp32
    assert oracle.swiglu(1.5, 2.0, 1.702, 1.0, lim) == pytest.approx(1.5 / (1 + math.exp(-a32 * 1.5)) * 3.0, rel=1e-15)


def test_geglu_tanh_pins():
    import torch
    # closed forms: zero gate, saturation on both sides
    assert oracle.geglu_tanh(0.0, 5.0) == 0.0
    assert oracle.geglu_tanh(40.0, 3.0) == 120.0
    assert abs(oracle.geglu_tanh(-40.0, 3.0)) < 1e-20
    xs = [float(np.float32(v)) for v in np.linspace(-6.0, 6.0, 97)]
    for x in xs:
        # gelu(x) - gelu(-x) = x holds for the tanh form (tanh is odd)
        assert oracle.geglu_tanh(x, 1.0) - oracle.geglu_tanh(-x, 1.0) == pytest.approx(x, rel=1e-14, abs=1e-15)
        # torch's tanh-approximate GELU (library routine), fp64
        want = float(torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh")) * 1.5
        assert oracle.geglu_tanh(x, 1.5) == pytest.approx(want, rel=1e-14, abs=1e-300)
        # and it stays within the approximation's error of the exact GELU x * Phi(x)
        assert abs(oracle.geglu_tanh(x, 1.0) - x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))) < 1e-3


def test_situ_pins():
    xs = [float(np.float32(v)) for v in np.linspace(-8.0, 8.0, 65)]
    for g in xs:
        # beta -> infinity: beta * tanh(g / beta) -> g, so SiTU is SwiGLU (silu(g) * u)
        assert oracle.situ(g, 1.25, 1e30) == pytest.approx(oracle.swiglu(g, 1.25), rel=1e-12, abs=1e-300)
        # the gate is bounded by beta
        assert abs(oracle.situ(g, 1.0, 0.5)) <= 0.5
        # the up-branch clamp is odd in u and bounded by its beta
        assert oracle.situ(g, -3.0, 0.5, 0.25) == -oracle.situ(g, 3.0, 0.5, 0.25)
        assert abs(oracle.situ(g, 1e6, 0.5, 0.25)) <= 0.5 * 0.25 * (1 + 1e-15)
    assert oracle.situ(0.0, 3.0, 0.5) == 0.0
    b = float(np.float32(0.5))
    # saturation: g >> beta gives beta * u, g << -beta gives ~0
    assert oracle.situ(40.0, 3.0, 0.5) == pytest.approx(b * 3.0, rel=1e-15)
    assert abs(oracle.situ(-40.0, 3.0, 0.5)) < 1e-16
    # small |g| and |u|: tanh(z) ~ z, the gate is ~ silu(g) and the clamp ~ identity
    assert oracle.situ(1e-4, 2e-4, 0.5, 0.25) == pytest.approx(oracle.swiglu(1e-4, 2e-4), rel=1e-6)


def _scaled_problem(mode, seed, up=True, per_token=False):
    p = _problem(mode, M=9, H=64, I=64, E=8, El=6, k=3, seed=seed, offset=1)
    rng = np.random.default_rng(seed)
    if up:
        p.w1_alpha_up = (p.w1_alpha * rng.uniform(0.5, 2.0, p.w1_alpha.shape)).astype(np.float32)
    if per_token:
        p.per_token_scale = rng.uniform(0.25, 4.0, p.M).astype(np.float32)
    return p


@pytest.mark.parametrize("mode,per_token", [(oracle.W4A16, False), (oracle.W4A4, True), (oracle.MXFP8_MXFP4, False)])
def test_separate_up_scale_and_per_token_scale(mode, per_token):
    """The up half's own per-expert scale and the W4A4 per-token input row
    scale: against the independent torch pipeline, and plan-based equal to
    per-token evaluation bit for bit."""
    p = _scaled_problem(mode, 61 + mode, up=True, per_token=per_token)
    tokens = np.arange(p.M)
    got = oracle.forward_tokens(p, tokens)
    _close_bf16(got, ref.forward_tokens(p, tokens))
    _, _, _, _, out = oracle.forward_plan(p, 4)
    assert np.array_equal(out, got)


def test_neutral_scales_change_nothing():
    # an up scale equal to w1_alpha, or a per-token scale of ones, is no scale at all
    for mode in (oracle.W4A16, oracle.W4A4):
        p = _problem(mode, M=8, H=64, I=64, E=4, El=4, k=2, seed=63)
        want = oracle.forward_tokens(p, np.arange(p.M))
        p.w1_alpha_up = p.w1_alpha.copy()
        if mode == oracle.W4A4:
            p.per_token_scale = np.ones(p.M, np.float32)
        assert np.array_equal(oracle.forward_tokens(p, np.arange(p.M)), want)


def test_power_of_two_up_scale_scales_y1_exactly():
    # SwiGLU at its defaults is linear in the up branch: doubling the up scale doubles y1 exactly
    p = _problem(oracle.W4A16, M=6, H=64, I=32, E=4, El=4, k=2, seed=64)
    _, y1, _, _, _ = oracle.forward_plan(p, 4)
    p.w1_alpha_up = (p.w1_alpha * np.float32(2.0)).astype(np.float32)
    plan, y1b, _, _, _ = oracle.forward_plan(p, 4)
    valid = plan.permuted_to_expanded >= 0
    assert np.array_equal(synth.bf16_to_f32(y1[valid]) * 2, synth.bf16_to_f32(y1b[valid]))


def _biased_problem(mode, seed):
    p = _problem(mode, M=9, H=64, I=64, E=8, El=6, k=3, seed=seed, offset=1)
    rng = np.random.default_rng(seed)
    p.fc1_bias = rng.normal(0.0, 0.05, (p.num_local_experts, 2 * p.I)).astype(np.float32)
    p.fc2_bias = rng.normal(0.0, 0.05, (p.num_local_experts, p.H)).astype(np.float32)
    return p


@pytest.mark.parametrize("mode", [oracle.W4A16, oracle.W4A4, oracle.MXFP8_MXFP4])
def test_fc_biases_against_library_reference(mode):
    p = _biased_problem(mode, 71 + mode)
    if mode == oracle.W4A4:
        oracle.set_fc2_input_scale(p, oracle.fc2_input_scale(p))
    tokens = np.arange(p.M)
    got = oracle.forward_tokens(p, tokens)
    _close_bf16(got, ref.forward_tokens(p, tokens))
    _, _, _, _, out = oracle.forward_plan(p, 4)
    assert np.array_equal(out, got)


def test_fc_biases_closed_forms():
    p = _biased_problem(oracle.W4A16, 74)
    plain = oracle.forward_tokens(_problem(oracle.W4A16, M=9, H=64, I=64, E=8, El=6, k=3, seed=74, offset=1),
                                  np.arange(p.M))
    zero = _biased_problem(oracle.W4A16, 74)
    zero.fc1_bias = np.zeros_like(zero.fc1_bias)
    zero.fc2_bias = np.zeros_like(zero.fc2_bias)
    assert np.array_equal(oracle.forward_tokens(zero, np.arange(p.M)), plain)   # zero biases are no biases
    # all-zero weight codes: the accumulators vanish, so y1 = bf16(silu(b_gate) * b_up) and y2 = bf16(b2)
    p.w1 = np.zeros_like(p.w1)
    p.w2 = np.zeros_like(p.w2)
    plan, y1, _, y2, _ = oracle.forward_plan(p, 4)
    for slot in np.nonzero(plan.permuted_to_expanded >= 0)[0]:
        le = int(p.topk_ids.reshape(-1)[plan.permuted_to_expanded[slot]]) - p.local_expert_offset
        bg, bu = p.fc1_bias[le, :p.I], p.fc1_bias[le, p.I:]
        want1 = ref.to_bf16_bits(np.array([oracle.swiglu(float(g), float(u)) for g, u in zip(bg, bu)]))
        assert np.array_equal(y1[slot], want1)
        assert np.array_equal(y2[slot], ref.to_bf16_bits(p.fc2_bias[le].astype(np.float64)))


def test_relu2_closed_forms():
    p = _problem(oracle.W4A16, M=6, H=64, I=32, E=4, El=4, k=2, seed=65, activation=oracle.ACT_RELU2)
    assert p.w1.shape[1] == p.I                 # non-gated: I rows of W1
    plan, y1, _, _, _ = oracle.forward_plan(p, 4)
    valid = plan.permuted_to_expanded >= 0
    v = synth.bf16_to_f32(y1[valid])
    assert np.all(v >= 0) and np.any(v == 0) and np.any(v > 0)
    # degree-2 homogeneity: doubling the expert scale quadruples y1 exactly
    p.w1_alpha = (p.w1_alpha * np.float32(2.0)).astype(np.float32)
    _, y1b, _, _, _ = oracle.forward_plan(p, 4)
    assert np.array_equal(v * 4, synth.bf16_to_f32(y1b[valid]))
    # all-zero weight codes with a bias: y1 = bf16(relu(b)^2) exactly
    p.w1 = np.zeros_like(p.w1)
    p.fc1_bias = np.random.default_rng(66).normal(0, 0.5, (p.num_local_experts, p.I)).astype(np.float32)
    plan, y1c, _, _, _ = oracle.forward_plan(p, 4)
    for slot in np.nonzero(plan.permuted_to_expanded >= 0)[0]:
        le = int(p.topk_ids.reshape(-1)[plan.permuted_to_expanded[slot]]) - p.local_expert_offset
        b = np.maximum(p.fc1_bias[le].astype(np.float64), 0.0)
        assert np.array_equal(y1c[slot], ref.to_bf16_bits(b * b))


def test_power_of_two_w2_alpha_scales_y2_exactly():
    p = _problem(oracle.W4A16, M=8, H=64, I=32, E=4, El=4, k=2, seed=32)
    _, _, _, y2, _ = oracle.forward_plan(p, 8)
    p.w2_alpha = (p.w2_alpha * np.float32(4.0)).astype(np.float32)
    _, _, _, y2b, _ = oracle.forward_plan(p, 8)
    a = synth.bf16_to_f32(y2)
    b = synth.bf16_to_f32(y2b)
    assert np.array_equal(a * 4, b)


def test_single_expert_single_route_is_a_plain_matmul_chain():
    # E_l = 1, top_k = 1: y2 = bf16(alpha2 * W2 . bf16(silu(alpha1 W1g . x) * alpha1 W1u . x)) via numpy matmul
    p = _problem(oracle.W4A16, M=6, H=64, I=32, E=1, El=1, k=1, seed=33)
    W1 = ref.deq_rows(p.mode, p.w1[0], p.w1_sf[0])
    W2 = ref.deq_rows(p.mode, p.w2[0], p.w2_sf[0])
    X = ref.bf16_vals(p.x)
    GU = (X @ W1.T).astype(np.float32) * np.float32(p.w1_alpha[0])
    y1 = ref.bf16_vals(ref.to_bf16_bits(ref.swiglu(GU[:, :32], GU[:, 32:], 1.0, 0.0, FLT_MAX)))
    Y = ((y1 @ W2.T).astype(np.float32) * np.float32(p.w2_alpha[0])).astype(np.float32)
    plan, y1o, _, y2o, out = oracle.forward_plan(p, 1)
    rows = plan.expanded_to_permuted
    assert np.mean(ref.bf16_vals(y1o[rows]) == y1) > 0.99
    np.testing.assert_allclose(ref.bf16_vals(y2o[rows]), Y, rtol=2 ** -7, atol=1e-12)


def test_requant_codes_of_plan_match_library_reference():
    # W4A4: the FC1 output is requantised to NVFP4 with fc2_input_scale; MX: to MXFP8
    p = _problem(oracle.W4A4, M=8, H=64, I=64, E=4, El=4, k=2, seed=34)
    plan, y1q, y1sf, _, _ = oracle.forward_plan(p, 4)
    t, j = 3, 1
    le = int(p.topk_ids[t, j])
    y1b, q, sf, a2 = oracle.gemm1_route(p, t, le)
    codes, scales, deq = ref.quant_nvfp4(ref.bf16_vals(y1b).astype(np.float32), p.fc2_input_scale)
    assert np.array_equal(ref.unpack(q), codes) and np.array_equal(sf, scales)
    np.testing.assert_array_equal(a2, deq)
    slot = plan.expanded_to_permuted[t * p.top_k + j]
    assert np.array_equal(y1q[slot], q) and np.array_equal(y1sf[slot], sf)


def test_fc2_calibration_is_max_over_all_routes():
    p = _problem(oracle.W4A4, M=6, H=64, I=32, E=4, El=4, k=2, seed=35)
    amax = 0.0
    for t in range(p.M):
        for j in range(p.top_k):
            y1b, _, _, _ = oracle.gemm1_route(p, t, int(p.topk_ids[t, j]))
            amax = max(amax, float(np.abs(synth.bf16_to_f32(y1b)).max()))
    assert p.fc2_input_scale == np.float32(amax) / np.float32(2688.0)
