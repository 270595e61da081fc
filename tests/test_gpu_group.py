"""Per-group dynamic quantisation (MoeDistributeDispatchV2 case 4) on the GPU.

The token and weight quantisers are compared bit for bit with the oracle's
(E4M3 codes and float32 descales): every decision is a float32 maximum, one
IEEE division, one float32 product and one round-to-nearest-even cast, taken
in the same precision on both sides.
"""

import numpy as np
import pytest

from _util import announce, bf16_tensor
from mixture_experts_ffn_int32_amd import synth
from oracle.quant import GROUP, quantize_columns_groups, quantize_rows_groups

pytestmark = pytest.mark.gpu


def _e4m3_values(q):
    import torch
    return q.cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _bf16_groups(shape, seed):
    """Normal values with a different magnitude per 128-group (2^-30 .. 2^30), 1% outliers
    x30, an all-zero group, a group of tiny values and one near the top of the bf16 range."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape).astype(np.float32)
    ng = shape[-1] // GROUP
    a *= np.repeat(np.exp2(rng.integers(-30, 30, shape[:-1] + (ng,))).astype(np.float32), GROUP, axis=-1)
    a[rng.random(shape) < 0.01] *= 30.0
    flat = a.reshape(-1, shape[-1])
    flat[0, :GROUP] = 0.0
    if flat.shape[0] > 2:
        flat[1, GROUP:2 * GROUP] *= 1e-25
        flat[2, :GROUP] = np.float32(2.0 ** 120) * np.sign(flat[2, :GROUP])
    return synth.to_bf16_bits(a)


@pytest.mark.parametrize("T,H", [(1, 128), (37, 384), (300, 4096), (5, 7168)])
def test_group_row_quantiser_bit_exact(T, H):
    from mixture_experts_ffn_int32_amd import quantize_rows_group as gpu_rows
    bits = _bf16_groups((T, H), seed=T + H)
    announce("group row quantiser T=%d H=%d" % (T, H))
    q, d = gpu_rows(bf16_tensor(bits, "cuda"))
    rq, _, rd = quantize_rows_groups(synth.bits_to_f32(bits))
    assert np.array_equal(d.cpu().numpy(), rd)
    assert np.array_equal(_e4m3_values(q), rq)


@pytest.mark.parametrize("E,H,N", [(1, 128, 64), (3, 384, 200), (2, 1024, 3072)])
def test_group_column_quantiser_bit_exact(E, H, N):
    from mixture_experts_ffn_int32_amd import quantize_cols_group as gpu_cols
    bits = _bf16_groups((E, N, H), seed=E + H + N).transpose(0, 2, 1).copy()   # blocks along H per column
    bits[:, :, 3] = 0                                                         # an all-zero column
    announce("group column quantiser E=%d H=%d N=%d" % (E, H, N))
    q, d = gpu_cols(bf16_tensor(bits, "cuda"))
    qv = _e4m3_values(q)
    dv = d.cpu().numpy()                       # [E, H/128, N]
    w = synth.bits_to_f32(bits)
    for e in range(E):
        rq, _, rd = quantize_columns_groups(w[e])
        assert np.array_equal(qv[e], rq), e
        assert np.array_equal(dv[e], rd), e


def test_group_quantisers_empty_and_repeatable():
    import torch
    from mixture_experts_ffn_int32_amd import quantize_cols_group as gpu_cols
    from mixture_experts_ffn_int32_amd import quantize_rows_group as gpu_rows
    announce("group quantisers T=0 and determinism")
    q, d = gpu_rows(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 256) and d.shape == (0, 2)
    bits = _bf16_groups((2, 64, 256), seed=5).transpose(0, 2, 1).copy()   # [E, H, N]
    w = bf16_tensor(bits, "cuda")
    a, b = gpu_cols(w), gpu_cols(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
