"""Pins of the oracle's number formats against things other than itself:
the OCP spec tables (tests/golden), torch's float8/bfloat16 conversions
(library routines) and brute-force nearest-value search over the tables."""
import math
import os

import numpy as np
import pytest
import torch

import oracle


def _read_table(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 0), float(v)))
    return rows


def test_e2m1_table_exhaustive(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_table.txt"))
    assert len(rows) == 16
    for code, value in rows:
        got = oracle.e2m1_value(code)
        assert got == value and math.copysign(1, got) == math.copysign(1, value), (code, got, value)


def test_e4m3_special_codes(golden_dir):
    for code, value in _read_table(os.path.join(golden_dir, "e4m3_special.txt")):
        got = oracle.e4m3_value(code)
        if math.isnan(value):
            assert math.isnan(got), code
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), (code, got, value)


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_value(c) for c in range(256)])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])


def _edge_doubles():
    v = [0.0, -0.0, 1.0, -1.0, 3.0e38, 3.4e38, 3.3895313892515355e38, 1e-40, -1e-40, 9.2e-41, 1.17549435e-38,
         2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 2.0 ** -126 * (1 + 2.0 ** -8)]
    # exact ties between neighbouring bf16 values (both parities)
    for m in (0x3f80, 0x3f81, 0x4049, 0x404a, 0xc123, 0x0001, 0x0080):
        lo = float(np.array([m << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(m + 1) << 16], np.uint32).view(np.float32)[0])
        v += [(lo + hi) / 2, np.nextafter((lo + hi) / 2, math.inf), np.nextafter((lo + hi) / 2, -math.inf)]
    return np.array(v, np.float64)


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        _edge_doubles().astype(np.float32),
    ])
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_round_single_rounding_from_double():
    # a double just above a bf16 tie must round up even where rounding it to
    # fp32 first would land on the tie and then go to even
    lo = float(np.array([0x3f80 << 16], np.uint32).view(np.float32)[0])   # 1.0
    ulp = 2.0 ** -7
    v = lo + ulp / 2 + 2.0 ** -40                                        # just above the tie
    assert oracle.bf16_round(np.array([v]))[0] == 0x3f81
    assert oracle.bf16_round(np.array([lo + ulp / 2]))[0] == 0x3f80      # tie -> even


def _brute_nearest_even(v, table_codes, table_vals, maxcode_val):
    """argmin |table - a| with ties to the even code, saturating at the max."""
    a = min(abs(v), maxcode_val)
    best = None
    for c, tv in zip(table_codes, table_vals):
        d = abs(tv - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return best[1]


def _test_values(rng, scale):
    v = np.concatenate([
        rng.standard_normal(3000) * scale,
        rng.uniform(-1, 1, 3000) * scale * 8,
        np.round(rng.uniform(-64, 64, 2000)) / 16 * scale,   # many exact ties
    ])
    return v.astype(np.float32)


def test_e2m1_encode_matches_brute_force(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_table.txt"))
    codes = [c for c, _ in rows[:8]]
    vals = [v for _, v in rows[:8]]
    rng = np.random.default_rng(1)
    v = np.concatenate([_test_values(rng, 2.0), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0,
                                                          6.0, 100.0, -0.0, 0.0, 1e-30], np.float32)])
    got = oracle.e2m1_encode(v)
    for x, g in zip(v, got):
        mag = _brute_nearest_even(float(x), codes, vals, 6.0)
        sign = 8 if math.copysign(1.0, float(x)) < 0 else 0
        assert g == (sign | mag), (x, g, sign | mag)


def test_e4m3_encode_matches_brute_force_and_torch():
    codes = list(range(127))
    vals = [oracle.e4m3_value(c) for c in codes]
    rng = np.random.default_rng(2)
    v = np.concatenate([_test_values(rng, 1.0), _test_values(rng, 100.0), _test_values(rng, 1e-3),
                        np.array([448.0, 449.0, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -9 * 1.5,
                                  0.0, -0.0], np.float32)])
    got = oracle.e4m3_encode(v)
    for x, g in zip(v, got):
        mag = _brute_nearest_even(float(x), codes, vals, 448.0)
        sign = 0x80 if math.copysign(1.0, float(x)) < 0 else 0
        assert g == (sign | mag), (x, g, sign | mag)
    # torch's fp32 -> e4m3fn conversion (round-to-nearest-even) agrees wherever it does not overflow
    inr = np.abs(v) < 464.0
    ref = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, got[inr])
