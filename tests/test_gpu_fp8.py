"""FP8 up-projection on the GPU.

The quantisers are compared bit for bit with the oracle's (codes and float32
descales): every decision they take is a float32 operation the pages fix.
The FP8 forward and the backward after it are compared with the FAITHFUL
oracle in its FP8 mode, element by element, in both tilings.
"""

import numpy as np
import pytest

from _util import announce, assert_close, bf16_tensor, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from oracle.quant import quantize_columns, quantize_rows
from oracle.routing import route as oracle_route
from test_gpu_parity import run_gpu

pytestmark = pytest.mark.gpu


def _e4m3_values(q):
    import torch
    return q.cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _bf16_matrix(shape, seed, outliers=True):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        m = rng.random(shape) < 0.01
        a[m] *= 40.0
        # values at the edge of the bf16 range of a row: tiny rows and huge rows
        a.reshape(-1, shape[-1])[1] *= 1e-30
        a.reshape(-1, shape[-1])[2] *= 1e30
    return synth.to_bf16_bits(a)


def _tiny(shape, seed):
    """bf16 values of magnitude up to ~1e-38 (bf16 subnormals included), a third of them zero."""
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(shape) * 4e-39).astype(np.float32)
    a[rng.random(shape) < 1 / 3] = 0
    return synth.to_bf16_bits(a)


@pytest.mark.parametrize("T,H", [(1, 64), (37, 320), (300, 4096)])
def test_row_quantiser_bit_exact(T, H):
    from mixture_experts_ffn_int32_amd import quantize_rows_fp8
    bits = _bf16_matrix((T, H), seed=T + H, outliers=T > 2)
    if T > 3:
        bits[3] = 0                              # an all-zero row: scale 1, codes 0
    if T > 4:
        # a row whose largest value (~1e-38, with zeros) makes 448 / max overflow float32:
        # the scale is clamped to the largest finite float32, the codes stay finite
        bits[4] = _tiny(bits[4].shape, seed=T)
    announce("row quantiser T=%d H=%d" % (T, H))
    q, ds = quantize_rows_fp8(bf16_tensor(bits, "cuda"))
    rq, _, rds = quantize_rows(synth.bits_to_f32(bits))
    assert np.array_equal(_e4m3_values(q), rq)
    assert np.array_equal(ds.cpu().numpy(), rds)


# the last case: many experts, H not a multiple of the 256-row chunks of the maxima,
# N not a multiple of a wave's 128 columns
@pytest.mark.parametrize("E,H,N", [(1, 64, 128), (3, 320, 192), (2, 1024, 3072), (6, 200, 3080)])
def test_column_quantiser_bit_exact(E, H, N):
    from mixture_experts_ffn_int32_amd import quantize_cols_fp8
    bits = _bf16_matrix((E, H, N), seed=E * H + N)
    bits[:, :, 5] = 0                            # an all-zero column in every expert
    bits[:, :, 7] = _tiny(bits[:, :, 7].shape, seed=E)   # a column whose 448 / max overflows float32
    announce("column quantiser E=%d H=%d N=%d" % (E, H, N))
    q, ds = quantize_cols_fp8(bf16_tensor(bits, "cuda"))
    qv = _e4m3_values(q)
    dsv = ds.cpu().numpy()
    w = synth.bits_to_f32(bits)
    for e in range(E):
        rq, _, rds = quantize_columns(w[e])
        assert np.array_equal(qv[e], rq), e
        assert np.array_equal(dsv[e], rds), e


FP8_SMALL = [
    ("tiny", dict(T=128, H=128, I=64, E=4, K=2)),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("zipf", dict(T=411, H=384, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    ("outliers", dict(T=520, H=256, I=320, E=3, K=2, routing="hot", outlier_frac=0.02, outlier_scale=30.0)),
    # many experts: on 64x64 tiles the launches spread the real tiles over the XCDs
    ("e1024", dict(T=512, H=128, I=64, E=1024, K=8, routing="zipf", zipf_s=0.6, n_empty=200)),
]


@pytest.mark.parametrize("tiles", ["large", "narrow"])
@pytest.mark.parametrize("name,over", FP8_SMALL, ids=[s[0] for s in FP8_SMALL])
def test_fp8_forward_backward_parity(name, over, tiles):
    from mixture_experts_ffn_int32_amd import saved_views
    spec = synth.spec_with("tiny", gmm1="fp8", **over)
    inp = synth.make_inputs(spec, seed=21)
    announce("fp8 parity %s %s tiles=%s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, tiles, gmm1="fp8")
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1="fp8")
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


def test_fp8_differs_from_bf16_and_autograd_works():
    """The FP8 option really changes the up-projection, and runs under autograd."""
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=256, H=256, I=128, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=8), "cuda")
    announce("fp8 vs bf16")
    x = g["x"].clone().requires_grad_(True)
    y8 = hyper_mega_moe(x, g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"],
                        gmm1_dtype="fp8")
    y16 = hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"])
    assert not torch.equal(y8, y16)
    rel = ((y8.float() - y16.float()).norm() / y16.float().norm()).item()
    assert rel < 0.1, rel                        # E4M3 keeps about 2 significant decimal digits
    y8.backward(g["dY"])
    y_raw, saved, dx, *_ = run_gpu(g, gmm1="fp8")
    assert torch.equal(y8, y_raw) and torch.equal(x.grad, dx)


def test_fp8_rejects_h_not_multiple_of_128():
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=64, H=192, I=64, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=9), "cuda")
    announce("fp8 H=192 rejected")
    with pytest.raises(ValueError):
        hyper_mega_moe(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"],
                       gmm1_dtype="fp8")
    torch.cuda.synchronize()
