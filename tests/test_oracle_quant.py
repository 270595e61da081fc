"""Pins of the oracle's dynamic FP8 E4M3 quantisation and of the FP8 up-projection."""

import numpy as np
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16
from oracle.quant import quantize_columns, quantize_rows


def test_row_quant_matches_torch_float32_ops_and_cast():
    rng = np.random.default_rng(0)
    x = round_bf16(rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    q, scale, descale = quantize_rows(x)
    tx = torch.from_numpy(x)
    tscale = torch.tensor(448.0, dtype=torch.float32) / tx.abs().amax(dim=1)
    assert np.array_equal(scale, tscale.numpy())
    tq = (tx * tscale[:, None]).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(q, tq)
    assert np.array_equal(descale, (1.0 / tscale).numpy())
    # the largest magnitude of every row lands on +-448
    assert np.all(np.abs(q).max(axis=1) == 448.0)


def test_column_quant_matches_torch_float32_ops_and_cast():
    rng = np.random.default_rng(1)
    w = round_bf16(rng.standard_normal((128, 96)) / 11.3).astype(np.float32)
    q, scale, descale = quantize_columns(w)
    tw = torch.from_numpy(w)
    tscale = torch.tensor(448.0, dtype=torch.float32) / tw.abs().amax(dim=0)
    assert np.array_equal(scale, tscale.numpy())
    assert np.array_equal(q, (tw * tscale[None, :]).to(torch.float8_e4m3fn).to(torch.float64).numpy())
    assert np.array_equal(descale, (1.0 / tscale).numpy())


def test_zero_row_gets_unit_scale():
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = -2.0
    q, scale, descale = quantize_rows(x)
    assert scale[0] == 1.0 and scale[2] == 1.0 and descale[0] == 1.0
    assert np.all(q[0] == 0) and q[1, 5] == -448.0


def test_fp8_up_projection_equals_bf16_when_quantisation_is_exact():
    """Rows and columns whose entries are +-2^j with max 1 quantise exactly (scale 448).

    Then (xq . wq) * (1/448) * (1/448) equals x . W1 up to the float32 rounding of
    1/448, so the FP8 and bf16 up-projections agree to ~1e-7 in pure mode.  Each
    column has its own maximum, so a misapplied per-column scale would show.
    """
    rng = np.random.default_rng(2)
    T, H, I, E, K = 6, 32, 8, 2, 2
    x = np.where(rng.random((T, H)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (T, H))
    x[:, 0] = 1.0
    W1 = np.where(rng.random((E, H, 2 * I)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (E, H, 2 * I))
    colmax = 2.0 ** -rng.integers(0, 3, (E, 1, 2 * I))
    W1 = W1 * colmax
    W1[:, 0, :] = colmax[:, 0, :]
    W2 = rng.standard_normal((E, I, H))
    ids = np.array([[0, 1]] * T)
    w = np.full((T, K), 0.5, np.float32)
    y8 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="fp8").forward()
    y16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16").forward()
    assert np.allclose(y8, y16, rtol=1e-6, atol=1e-6)


def test_fp8_up_projection_error_is_bounded():
    """Generic data: each E4M3 code has relative error <= 2^-4, so h moves by a bounded amount."""
    rng = np.random.default_rng(3)
    T, H, I, E, K = 8, 64, 16, 3, 2
    x = round_bf16(rng.standard_normal((T, H)))
    W1 = round_bf16(rng.standard_normal((E, H, 2 * I)) / 8)
    W2 = round_bf16(rng.standard_normal((E, I, H)) / 4)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    w = np.full((T, K), 0.5, np.float32)
    m8 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="fp8")
    m16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")
    for e in range(E):
        h8 = m8.up(e, x)
        h16 = m16.up(e, x)
        bound = (2 * 2.0 ** -4 + 2.0 ** -8) * (np.abs(x) @ np.abs(W1[e]))
        assert np.all(np.abs(h8 - h16) <= bound)
