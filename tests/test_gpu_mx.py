"""MX up-projection (MoeDistributeDispatchV2 case 5) on the GPU.

The MX quantisers are compared bit for bit with the oracle's (codes and block
exponents): every decision is exact (a power-of-two scaling, then one
saturating round to E4M3).  The MX forward and the backward after it are
compared with the FAITHFUL oracle in its MX mode, element by element, in both
tilings, and sampled at full size.
"""

import numpy as np
import pytest

from _util import announce, assert_close, bf16_tensor, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from oracle.quant import quantize_columns_mx, quantize_rows_mx
from oracle.routing import route as oracle_route
from test_gpu_parity import run_gpu

pytestmark = pytest.mark.gpu


def _e4m3_values(q):
    import torch
    return q.cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _bf16_blocks(shape, seed):
    """Normal values with a different magnitude per 32-block (2^-40 .. 2^40), 1% outliers,
    some all-zero blocks and blocks near the ends of the bf16 range."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape).astype(np.float32)
    nb = shape[-1] // 32
    mag = np.exp2(rng.integers(-40, 40, shape[:-1] + (nb,))).astype(np.float32)
    a *= np.repeat(mag, 32, axis=-1)
    a[rng.random(shape) < 0.01] *= 30.0
    flat = a.reshape(-1, shape[-1])
    flat[0, :32] = 0.0
    if flat.shape[0] > 2:
        flat[1, 32:64] *= 1e-25
        flat[2, :32] = np.float32(2.0 ** 126) * np.sign(flat[2, :32])
    return synth.to_bf16_bits(a)


@pytest.mark.parametrize("T,H", [(1, 128), (37, 384), (300, 4096)])
def test_mx_row_quantiser_bit_exact(T, H):
    from mixture_experts_ffn_int32_amd import quantize_rows_mx as gpu_rows
    bits = _bf16_blocks((T, H), seed=T + H)
    announce("mx row quantiser T=%d H=%d" % (T, H))
    q, s = gpu_rows(bf16_tensor(bits, "cuda"))
    rq, re = quantize_rows_mx(synth.bits_to_f32(bits))
    assert np.array_equal(s.cpu().numpy().astype(np.int64) - 127, re)
    assert np.array_equal(_e4m3_values(q), rq)


@pytest.mark.parametrize("E,H,N", [(1, 128, 64), (3, 384, 192), (2, 1024, 3072)])
def test_mx_column_quantiser_bit_exact(E, H, N):
    from mixture_experts_ffn_int32_amd import quantize_cols_mx as gpu_cols
    rng = np.random.default_rng(E * H + N)
    bits = _bf16_blocks((E, N, H), seed=E + H + N).transpose(0, 2, 1).copy()   # blocks along H per column
    bits[:, :, 3] = 0                               # an all-zero column
    announce("mx column quantiser E=%d H=%d N=%d" % (E, H, N))
    q, s = gpu_cols(bf16_tensor(bits, "cuda"))
    qv = _e4m3_values(q)
    sv = s.cpu().numpy().astype(np.int64) - 127     # [E, N, H/32]
    w = synth.bits_to_f32(bits)
    for e in range(E):
        rq, re = quantize_columns_mx(w[e])          # [H, N], [H/32, N]
        assert np.array_equal(qv[e], rq), e
        assert np.array_equal(sv[e], re.T), e
    del rng


MX_SMALL = [
    ("tiny", dict(T=128, H=128, I=64, E=4, K=2)),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("zipf", dict(T=411, H=384, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    ("outliers", dict(T=520, H=256, I=320, E=3, K=2, routing="hot", outlier_frac=0.02, outlier_scale=30.0)),
]


@pytest.mark.parametrize("tiles", ["large", "narrow"])
@pytest.mark.parametrize("name,over", MX_SMALL, ids=[s[0] for s in MX_SMALL])
def test_mx_forward_backward_parity(name, over, tiles):
    from mixture_experts_ffn_int32_amd import saved_views
    spec = synth.spec_with("tiny", gmm1="mx", **over)
    inp = synth.make_inputs(spec, seed=23)
    announce("mx parity %s %s tiles=%s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, tiles, gmm1="mx")
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1="mx")
    v = saved_views(saved, *(spec[k] for k in "THIEK"), tiles=tiles)
    ref_route = oracle_route(inp["topk_ids"], spec["E"])
    (h, a, _), (hd, ad, _) = o.slot_intermediates_dev(ref_route["sorted_slot"])
    assert_close(to_f64(v["h"]), h, name + " h", hd)
    assert_close(to_f64(v["a"]), a, name + " a", ad)
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, name + " y", ryd)
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    assert_close(to_f64(dx), rdx, name + " dx", ddx)
    assert_close(to_f64(dw), rdw, name + " d_topk_weights", ddw)
    assert_close(to_f64(dW1), rdW1, name + " d_up_proj_weight", ddW1)
    assert_close(to_f64(dW2), rdW2, name + " d_down_proj_weight", ddW2)


def test_mx_differs_from_fp8_and_autograd_works():
    """MX really changes the up-projection (against per-token FP8 and bf16), and runs under autograd."""
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=256, H=256, I=128, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=10), "cuda")
    announce("mx vs fp8 vs bf16")
    x = g["x"].clone().requires_grad_(True)
    args = (g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    ymx = hyper_mega_moe(x, *args, gmm1_dtype="mx")
    y8 = hyper_mega_moe(g["x"], *args, gmm1_dtype="fp8")
    y16 = hyper_mega_moe(g["x"], *args)
    assert not torch.equal(ymx, y8) and not torch.equal(ymx, y16)
    rel = ((ymx.float() - y16.float()).norm() / y16.float().norm()).item()
    assert rel < 0.1, rel
    ymx.backward(g["dY"])
    y_raw, saved, dx, *_ = run_gpu(g, gmm1="mx")
    assert torch.equal(ymx, y_raw) and torch.equal(x.grad, dx)


def test_mx_with_shared_expert():
    """MX routed up-projection with a shared expert (whose up-projection stays bf16)."""
    from test_gpu_shared import check_all, run_shared
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3, gmm1="mx", shared_I=128)
    inp = synth.make_inputs(spec, seed=24)
    announce("mx + shared")
    g = gpu_inputs(inp, "cuda")
    got = run_shared(g, "auto", gmm1="mx")
    check_all("mx shared", MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1="mx"), got)


@pytest.mark.slow
def test_full_size_mx_sampled():
    """The MX workload (T=16384, H=4096, I=1536, E=64, K=6) on sampled tokens and columns."""
    from test_gpu_parity import _sample_full
    _sample_full("mx", n_tok=4)
