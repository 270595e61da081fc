"""Pins of the oracle's rounding primitives against library routines and closed forms."""

import numpy as np
import torch

from oracle.numerics import (BF16_MAX, E4M3_MAX, bf16_bits_to_f64, round_bf16, round_e4m3,
                             sigmoid, silu)


def _random_finite_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_bf16_matches_torch_on_random_float32():
    v = _random_finite_f32(1 << 20, 0)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(v.astype(np.float64))
    same = (got == ref) | (np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref)))
    assert same.all()


def test_bf16_ties_and_edges_match_torch():
    # exact ties (low 16 bits = 0x8000), values next to ties, subnormals, the top of the range
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << np.uint32(16)
    cases = np.concatenate([hi | np.uint32(0x8000), hi | np.uint32(0x7FFF), hi | np.uint32(0x8001),
                            hi | np.uint32(1), hi]).view(np.float32)
    cases = cases[np.isfinite(cases)]
    ref = torch.from_numpy(cases).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(cases.astype(np.float64))
    same = (got == ref) | (np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref)))
    assert same.all()


def test_bf16_rounds_float64_once():
    # 1 + 2^-8 + 2^-40 lies just above the bf16 tie between 1 and 1 + 2^-7; a detour
    # through float32 would turn it into the exact tie and round down to 1.
    assert round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert round_bf16(np.array([BF16_MAX]))[0] == BF16_MAX
    assert np.isinf(round_bf16(np.array([2.0 ** 128]))[0])
    assert round_bf16(np.array([-0.0]))[0] == 0.0


def test_bf16_bits_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-464, 464, 200000),
        rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000),
    ]).astype(np.float32)
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = round_e4m3(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_codes_are_fixed_points_and_saturate():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(round_e4m3(vals), vals)
    assert vals.max() == E4M3_MAX
    assert round_e4m3(np.array([1000.0, -1e6]))[0] == E4M3_MAX
    assert round_e4m3(np.array([-1e6]))[0] == -E4M3_MAX
    # the smallest subnormal is 2^-9; half of it is a tie and goes to zero
    assert round_e4m3(np.array([2.0 ** -10]))[0] == 0.0
    assert round_e4m3(np.array([1.5 * 2.0 ** -10]))[0] == 2.0 ** -9


def test_silu_sigmoid_match_torch():
    g = np.linspace(-40, 40, 10001)
    tg = torch.from_numpy(g)
    assert np.allclose(sigmoid(g), torch.sigmoid(tg).numpy(), rtol=1e-15, atol=1e-300)
    assert np.allclose(silu(g), torch.nn.functional.silu(tg).numpy(), rtol=1e-14, atol=1e-300)
