"""The seeded input generator: determinism, the SplitMix64 definition, the
distributions of the recipe and the router's properties."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the published generator
    # (state += 0x9E3779B97F4A7C15, then the finaliser) for seed 0
    state = 0
    outs = []
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) & (2 ** 64 - 1)
        outs.append(synth.lib().synth_mix64(state))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_determinism_and_streams():
    a = synth.normal_bf16(3, 1, (64, 64))
    b = synth.normal_bf16(3, 1, (64, 64))
    c = synth.normal_bf16(3, 2, (64, 64))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # a prefix of a longer draw is the shorter draw (counter-based)
    d = synth.normal_f32(3, 1, (10,))
    e = synth.normal_f32(3, 1, (1000,))
    assert np.array_equal(d, e[:10])


def test_normal_moments():
    v = synth.normal_f32(0, 7, (1 << 20,), 0.0, 0.02).astype(np.float64)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4
    x = synth.bf16_to_f32(synth.normal_bf16(0, 8, (1 << 18,))).astype(np.float64)
    assert abs(x.mean()) < 1e-2 and abs(x.std() - 1.0) < 1e-2


def test_router_properties():
    wl = synth.WORKLOADS["w4a16_prefill"]
    logits = synth.normal_f32(0, 2, (300, 256))
    bias = synth.normal_f32(0, 3, (256,), 0.0, 0.5)
    ids, w = synth.router(logits, bias, 8)
    z = logits.astype(np.float64) + bias
    for t in range(300):
        order = np.lexsort((np.arange(256), -z[t]))[:8]
        assert np.array_equal(ids[t], order)
        assert len(set(ids[t])) == 8
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_sample_tokens():
    s = synth.sample_tokens(4, 65536, 1024)
    assert s.size == 1024 and np.unique(s).size == 1024 and s[0] == 0 and s[-1] == 65535
    assert np.all(np.diff(s) > 0)
