"""Pins for the oracle's BF16 and E4M3 codecs.

Library routine: torch's bfloat16 and float8_e4m3fn conversions (CPU).
Published table: OCP OFP8 rev. 1.0, Table 1 (tests/golden/e4m3_ocp_table.txt).
Hand-worked ties-to-even cases (tests/golden/bf16_rne_cases.txt).
"""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_bits_to_f64, f64_to_bf16_bits, e4m3_to_f64, f64_to_e4m3


def _read_golden(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_bf16_encode_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x32 = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-39).astype(np.float32),   # subnormals
        # exact midpoints between neighbouring BF16 values
        ((rng.integers(0, 0x7F00, 50_000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    ours = f64_to_bf16_bits(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_hand_cases(golden_dir):
    for inp, bits in _read_golden(os.path.join(golden_dir, "bf16_rne_cases.txt")):
        got = int(f64_to_bf16_bits(np.float64(float(inp))))
        assert got == int(bits, 16), (inp, hex(got), bits)


def test_bf16_encode_nan_and_inf():
    out = f64_to_bf16_bits(np.array([np.nan, np.inf, -np.inf]))
    assert out.tolist() == [0x7FC0, 0x7F80, 0xFF80]


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zero is kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_ocp_table(golden_dir):
    for code, value in _read_golden(os.path.join(golden_dir, "e4m3_ocp_table.txt")):
        c = int(code, 16)
        got = float(e4m3_to_f64(np.uint8(c)))
        if value == "nan":
            assert np.isnan(got)
            continue
        v = float(value)
        assert got == v and np.signbit(got) == np.signbit(v), (code, got, value)
        # the encoder maps the value back to the same code
        assert int(f64_to_e4m3(np.float64(v))) == c


def test_e4m3_encode_matches_torch_below_overflow():
    """Dense sweep of |x| < 464 (where torch's RNE does not overflow to NaN)."""
    rng = np.random.default_rng(1)
    grid = np.linspace(-463.9, 463.9, 400_001)
    rnd = np.concatenate([rng.standard_normal(100_000) * s for s in (1e-3, 1.0, 30.0, 200.0)])
    # exact midpoints between neighbouring E4M3 values (ties to even)
    vals = np.unique(e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([grid, rnd, mids, -mids]).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) < 464.0]
    ours = f64_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_ties_to_even_hand_cases():
    # spacing 0.125 in [1, 2): 1.0625 is a tie between 1.0 (even) and 1.125
    cases = {1.0625: 1.0, 1.1875: 1.25, 17.0: 16.0, 19.0: 20.0, 464.0: 448.0}
    for x, want in cases.items():
        assert e4m3_to_f64(f64_to_e4m3(np.float64(x))) == want


def test_e4m3_clamps_instead_of_nan():
    """Reading R9: out-of-range values saturate to +-448; NaN stays NaN."""
    out = f64_to_e4m3(np.array([480.0, 1e9, -1e9, np.inf, -np.inf, np.nan]))
    assert out.tolist() == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_encode_output_by_hand():
    """R21 on hand-worked values (OCP E4M3: bias 7, 3 mantissa bits, max 448,
    subnormal step 2^-9), out_scale 2."""
    o = np.array([1.0, -1.0, 1000.0, -1000.0, 2.0 ** -4, 2.0 ** -8, 2.0 ** -11, 0.0,
                  2 * 1.0625, 2 * 1.1875, 2 * 3 * 2.0 ** -10])
    codes = oracle.encode_output(o, "fp8", 2.0)
    # 0.5 -> 0x30; 500 -> clamp 448 -> 0x7E; 2^-5 -> 0x10; 2^-9 -> 0x01 (smallest
    # subnormal); 2^-12 -> rounds to 0; 1.0625 (tie between 1 and 1.125) -> even 1.0 = 0x38;
    # 1.1875 (tie between 1.125 and 1.25) -> even 1.25 = 0x3A; 3*2^-10 = 1.5 subnormal
    # steps (tie) -> even 2 steps = 0x02
    assert codes.tolist() == [0x30, 0xB0, 0x7E, 0xFE, 0x10, 0x01, 0x00, 0x00, 0x38, 0x3A, 0x02]
    bits = oracle.encode_output(np.array([1.0, -2.5]), "bf16")
    assert bits.tolist() == [0x3F80, 0xC020]
    with pytest.raises(ValueError):
        oracle.encode_output(o, "fp16")
