"""Pins of the oracle's NVFP4 and MX quantisers: round trips of exactly
representable inputs, nearest-grid optimality by brute force, the range the
MX rule puts each block's amax in, and torch's e4m3 conversion."""
import math

import numpy as np
import torch

import oracle
import synth

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_vals(codes):
    codes = np.asarray(codes).astype(np.int64)
    v = E2M1[codes & 7]
    return np.where(codes & 8, -v, v)


def unpack(q, n):
    q = np.asarray(q, np.uint8)
    lo = q & 15
    hi = q >> 4
    return np.stack([lo, hi], -1).reshape(q.shape[:-1] + (2 * q.shape[-1],))[..., :n]


def e4m3_vals(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_nvfp4_round_trip_of_representable_blocks():
    rng = np.random.default_rng(3)
    rows, cols = 64, 128
    gs = np.float32(2.0 ** -7)   # a power of two keeps every product exact
    # choose scale codes and element codes; each block's largest element is
    # +-6 so that blockamax / (6 gs) is exactly the decoded scale
    sc = rng.integers(0x20, 0x6f, (rows, cols // 16)).astype(np.uint8)
    el = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    el[:, ::16] = np.where(rng.random((rows, cols // 16)) < 0.5, 7, 15)
    sd = e4m3_vals(sc).astype(np.float32)
    v = (e2m1_vals(el).astype(np.float32) * np.repeat(sd * gs, 16, axis=1)).astype(np.float32)
    q, s = oracle.nvfp4_quantize(v, gs)
    deq = e2m1_vals(unpack(q, cols)) * np.repeat(e4m3_vals(s), 16, 1) * np.float64(gs)
    assert np.array_equal(s, sc)
    # element codes: equal up to the sign of zero
    got = unpack(q, cols)
    assert np.array_equal(got & 7, el & 7)
    assert np.allclose(deq, v.astype(np.float64), rtol=0, atol=0)


def test_nvfp4_elements_are_nearest_grid_points():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((50, 64)) * rng.uniform(0.01, 3.0, (50, 1))).astype(np.float32)
    gs = np.float32(oracle.nvfp4_global_scale(float(np.abs(v).max())))
    q, s = oracle.nvfp4_quantize(v, gs)
    sd = e4m3_vals(s).astype(np.float32)
    denom = (np.repeat(sd, 16, 1) * gs).astype(np.float32)        # the fp32 decision quantity
    r = (v / denom).astype(np.float32)
    codes = unpack(q, 64)
    got = np.abs(e2m1_vals(codes))
    # brute force: distance to every magnitude, ties to the even code
    d = np.abs(np.abs(r)[..., None] - E2M1[None, None, :])
    d = np.where(np.abs(r)[..., None] >= 6.0, np.where(np.arange(8) == 7, 0.0, 1.0), d)
    best = np.argmin(d + (np.arange(8) % 2) * 1e-12, axis=-1)
    assert np.array_equal(E2M1[best], got)
    assert np.array_equal(codes >> 3, np.signbit(r).astype(np.uint8))


def test_nvfp4_block_scale_puts_block_max_near_six():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((200, 64)).astype(np.float32)
    gs = np.float32(oracle.nvfp4_global_scale(float(np.abs(v).max())))
    q, s = oracle.nvfp4_quantize(v, gs)
    bam = np.abs(v).reshape(200, 4, 16).max(-1)
    sd = e4m3_vals(s)
    ratio = bam / (sd * np.float64(gs))
    # E4M3 normal rounding changes the scale by at most 2^-4 relative
    normal = s >= 0x08
    assert np.all(np.abs(ratio[normal] - 6.0) <= 6.0 * 2.0 ** -4 * 1.0001)
    # the largest block of the tensor lands exactly on scale 448
    assert s.max() == 0x7e


def test_nvfp4_zero_block_and_global_scale():
    v = np.zeros((2, 32), np.float32)
    v[1, 16:] = np.linspace(-1, 1, 16)
    q, s = oracle.nvfp4_quantize(v, np.float32(1.0 / 2688))
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and np.all(q[0] == 0)
    assert oracle.nvfp4_global_scale(2688.0) == 1.0


def test_mx_block_exponent_rule():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((100, 64)) * np.exp(rng.uniform(-20, 20, (100, 1)))).astype(np.float32)
    for elem, emax in ((oracle.ELEM_E4M3, 8), (oracle.ELEM_E2M1, 2)):
        q, s = oracle.mx_quantize(v, elem)
        amax = np.abs(v).reshape(100, 2, 32).max(-1).astype(np.float64)
        X = 2.0 ** (s.astype(np.float64) - 127)
        r = amax / X
        assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1))), elem


def test_mx_e4m3_elements_match_torch_with_saturation():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    q, s = oracle.mx_quantize(v, oracle.ELEM_E4M3)
    X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, 1)
    r = (v / X).astype(np.float32)                # exact: X is a power of two
    ref = torch.from_numpy(np.clip(r, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, q)


def test_mx_e2m1_round_trip_and_nearest():
    rng = np.random.default_rng(8)
    rows, cols = 32, 64
    el = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    el[:, ::32] = 7          # block max exactly 6 = 1.5 * 2^2
    e = rng.integers(100, 150, (rows, cols // 32))
    v = (e2m1_vals(el) * np.repeat(2.0 ** (e - 127.0), 32, 1)).astype(np.float32)
    q, s = oracle.mx_quantize(v, oracle.ELEM_E2M1)
    assert np.array_equal(s.astype(np.int64), e)
    assert np.array_equal(unpack(q, cols) & 7, el & 7)


def test_quantize_bf16_wrappers_global_scale():
    x = synth.normal_bf16(11, 1, (8, 64))
    q, s, gs = oracle.nvfp4_quantize_bf16(x)
    f = synth.bf16_to_f32(x)
    assert gs == np.float32(np.abs(f).max()) / np.float32(2688.0)
    q2, s2 = oracle.nvfp4_quantize(f, gs)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    qm, sm = oracle.mx_quantize_bf16(x, oracle.ELEM_E4M3)
    qm2, sm2 = oracle.mx_quantize(f, oracle.ELEM_E4M3)
    assert np.array_equal(qm, qm2) and np.array_equal(sm, sm2)
