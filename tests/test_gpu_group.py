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
    x30, an all-zero group, groups of tiny values (one whose 448 / max overflows float32) and
    one near the top of the bf16 range."""
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
    if flat.shape[0] > 3:
        # a group whose largest value (~1e-38, with zeros) makes 448 / max overflow float32
        flat[3, :GROUP] = rng.standard_normal(GROUP).astype(np.float32) * np.float32(4e-39)
        flat[3, :GROUP:3] = 0.0
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


# ----------------------------------------------------------------------------- the per-group up-projection
from _util import assert_close, gpu_inputs, oracle_inputs, to_f64  # noqa: E402
from oracle.moe_ffn import MoEFFN  # noqa: E402
from oracle.routing import route as oracle_route  # noqa: E402
from test_gpu_parity import _sample_full, run_gpu  # noqa: E402

GROUP_SMALL = [
    ("tiny", dict(T=128, H=128, I=64, E=4, K=2)),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("zipf", dict(T=411, H=384, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    ("outliers", dict(T=520, H=256, I=320, E=3, K=2, routing="hot", outlier_frac=0.02, outlier_scale=30.0)),
    # expert sizes of one to five 64-row entries, full and partial (the product's
    # 128-row tiles take the entries in pairs)
    ("bounds", dict(T=1092, H=256, I=64, E=9, K=1, routing="counts",
                    counts=[0, 1, 64, 65, 128, 129, 192, 193, 320])),
]


@pytest.mark.parametrize("tiles", ["narrow", "large"])
@pytest.mark.parametrize("name,over", GROUP_SMALL, ids=[s[0] for s in GROUP_SMALL])
def test_group_forward_backward_parity(name, over, tiles):
    """Forward intermediates, y and the whole backward against the FAITHFUL oracle in its
    per-group mode.  The up-projection always runs on 64-row tiles; with large tiles the
    other products run on 256-row tiles and a second routing pass writes its table."""
    from mixture_experts_ffn_int32_amd import saved_views
    spec = synth.spec_with("tiny", gmm1="group", **over)
    inp = synth.make_inputs(spec, seed=29)
    announce("group parity %s %s tiles %s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, tiles, gmm1="group")
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1="group")
    v = saved_views(saved, *(spec[k] for k in "THIEK"), tiles=tiles, gmm1_dtype="group")
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


def test_group_differs_from_per_token_and_tilings_agree():
    """Per-group scales change the up-projection against per-token FP8 (groups of very
    different magnitude); both tilings give the same forward bit for bit (the per-group
    product runs on 64-row tiles in both, and the down-projection's sums do not depend on
    the row tiling)."""
    spec = synth.spec_with("tiny", T=256, H=512, I=128, E=4, K=2)
    inp = synth.make_inputs(spec, seed=31)
    inp["x"] = synth.to_bf16_bits(synth.bits_to_f32(inp["x"]) *
                                  np.repeat(np.exp2(np.arange(4) * 6.0 - 9.0), GROUP)[None, :].astype(np.float32))
    announce("group against per-token")
    g = gpu_inputs(inp, "cuda")
    y_g = run_gpu(g, "narrow", gmm1="group")[0]
    y_t = run_gpu(g, "narrow", gmm1="fp8")[0]
    assert not np.array_equal(to_f64(y_g), to_f64(y_t))
    y_l = run_gpu(g, "large", gmm1="group")[0]
    assert np.array_equal(to_f64(y_g), to_f64(y_l))


def test_full_size_group_sampled():
    """The FP8-size workload with per-group scales, sampled (as the other full-size tests)."""
    _sample_full("group")
