"""The float32-output (accuracy) mode against the PURE oracle (no intermediate rounding).

The bar is the RFC's 1e-3 (section 7.1): |gpu - ref| <= 1e-3 + 1e-3 |ref| on every
element of y, dx, d_topk_weights, dW1 and dW2, with dY a float32 tensor that is
not bf16-representable (so its low half is exercised too).
"""

import numpy as np
import pytest

from _util import announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from oracle.routing import route as oracle_route

pytestmark = pytest.mark.gpu

TOL = 1e-3


def f32_dy(inp, seed):
    """dY in float32 that bf16 cannot hold: the bf16 draw times (1 + 1e-3 N(0,1))."""
    rng = np.random.default_rng(seed)
    d = synth.bits_to_f32(inp["dY"])
    return (d * (1.0 + 1e-3 * rng.standard_normal(d.shape))).astype(np.float32)


def run_f32(g, dy, tiles):
    import torch
    from mixture_experts_ffn_int32_amd import backward_from_saved, forward_with_saved
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], tiles=tiles, out_dtype="f32")
    dx, dW1, dW2, dw = backward_from_saved(dy, g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                           g["down_proj_weight"], saved, tiles=tiles, out_dtype="f32")
    torch.cuda.synchronize()
    assert y.dtype == dx.dtype == dW1.dtype == dW2.dtype == torch.float32
    return y, saved, dx, dW1, dW2, dw


CASES = [
    ("tiny", dict()),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("hot", dict(T=257, H=192, I=128, E=5, K=2, routing="hot")),
    ("zipf", dict(T=411, H=256, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
]


@pytest.mark.parametrize("tiles", ["large", "narrow"])
@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_f32_mode_matches_pure_oracle(name, over, tiles):
    import torch
    spec = synth.spec_with("tiny", **over)
    inp = synth.make_inputs(spec, seed=31)
    announce("f32 mode %s %s tiles=%s" % (name, {k: spec[k] for k in "THIEK"}, tiles))
    g = gpu_inputs(inp, "cuda")
    dy = f32_dy(inp, 5)
    y, saved, dx, dW1, dW2, dw = run_f32(g, torch.from_numpy(dy).cuda(), tiles)
    oi = oracle_inputs(inp)
    oi["dY"] = dy
    o = MoEFFN(**oi, mode="pure")
    ry, _ = o.forward_dev(out_dtype="f32")
    assert_close(to_f64(y), ry, name + " y", rtol=TOL, atol=TOL)
    (rdx, rdw, rdW1, rdW2), _ = o.backward_dev(out_dtype="f32")
    assert_close(to_f64(dx), rdx, name + " dx", rtol=TOL, atol=TOL)
    assert_close(to_f64(dw), rdw, name + " d_topk_weights", rtol=TOL, atol=TOL)
    assert_close(to_f64(dW1), rdW1, name + " d_up_proj_weight", rtol=TOL, atol=TOL)
    assert_close(to_f64(dW2), rdW2, name + " d_down_proj_weight", rtol=TOL, atol=TOL)
    counts = np.bincount(inp["topk_ids"].reshape(-1), minlength=spec["E"])
    for e in np.flatnonzero(counts == 0):
        assert not to_f64(dW1[e]).any() and not to_f64(dW2[e]).any()


def test_f32_mode_intermediates():
    """h in float32 and a as hi + lo agree with the unrounded values to ~16 bits."""
    from mixture_experts_ffn_int32_amd import saved_views
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3)
    inp = synth.make_inputs(spec, seed=33)
    announce("f32 mode intermediates")
    g = gpu_inputs(inp, "cuda")
    import torch
    y, saved, *_ = run_f32(g, torch.from_numpy(f32_dy(inp, 6)).cuda(), "large")
    T, H, I, E, K = (spec[k] for k in "THIEK")
    v = saved_views(saved, T, H, I, E, K, tiles="large", out_dtype="f32")
    ref_route = oracle_route(inp["topk_ids"], E)
    o = MoEFFN(**oracle_inputs(inp), mode="pure")
    (h, a, _), _ = o.slot_intermediates_dev(ref_route["sorted_slot"])
    assert_close(to_f64(v["h"]), h, "h", rtol=1e-5, atol=1e-5)
    a2 = to_f64(v["a"])
    assert_close(a2[:, :I] + a2[:, I:], a, "a hi + lo", rtol=2e-5, atol=1e-6)
    assert np.array_equal(a2[:, :I], to_f64(torch.from_numpy(a2[:, :I].astype(np.float32)).bfloat16()))


def test_f32_mode_autograd_and_determinism():
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=96, H=128, I=64, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=34), "cuda")
    announce("f32 mode autograd")
    x = g["x"].clone().requires_grad_(True)
    y = hyper_mega_moe(x, g["topk_ids"], g["topk_weights"], g["up_proj_weight"], g["down_proj_weight"],
                       out_dtype=torch.float32)
    assert y.dtype == torch.float32
    dy = torch.randn(y.shape, device="cuda", dtype=torch.float32)
    y.backward(dy)
    r1 = run_f32(g, dy, "auto")
    r2 = run_f32(g, dy, "auto")
    assert torch.equal(y, r1[0]) and torch.equal(x.grad, r1[2].to(torch.bfloat16))
    for i in (0, 2, 3, 4, 5):
        assert torch.equal(r1[i], r2[i])


@pytest.mark.slow
def test_f32_mode_skewed_sampled():
    """The skewed workload (big and small tiles, empty and tiny experts) in the accuracy mode, sampled."""
    import torch
    spec = synth.WORKLOADS["skewed"]
    T, H, I, E, K = (spec[k] for k in "THIEK")
    inp = synth.make_inputs(spec, seed=0)
    announce("f32 mode skewed sampled")
    g = gpu_inputs(inp, "cuda")
    dy = f32_dy(inp, 7)
    y, saved, dx, dW1, dW2, dw = run_f32(g, torch.from_numpy(dy).cuda(), "auto")
    oi = oracle_inputs(inp)
    oi["dY"] = dy
    o = MoEFFN(**oi, mode="pure")
    rng = np.random.default_rng(2)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 5, replace=False)]))
    ti = torch.from_numpy(toks).cuda()
    ry, _ = o.forward_dev(toks, out_dtype="f32")
    assert_close(to_f64(y[ti]), ry, "skewed f32 y", rtol=TOL, atol=TOL)
    (rdx, rdw), _ = o.backward_tokens_dev(toks, out_dtype="f32")
    assert_close(to_f64(dx[ti]), rdx, "skewed f32 dx", rtol=TOL, atol=TOL)
    assert_close(to_f64(dw[ti]), rdw, "skewed f32 d_topk_weights", rtol=TOL, atol=TOL)
    counts = np.bincount(inp["topk_ids"].reshape(-1), minlength=E)
    nz = np.flatnonzero(counts)
    icols = np.array([0, I // 3, I - 1])
    for e in sorted({int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])}):
        (gc, uc, dr), _ = o.weight_grads_expert_dev(e, icols, out_dtype="f32")
        assert_close(to_f64(dW1[e][:, icols]), gc, "skewed f32 dW1[%d] gate" % e, rtol=TOL, atol=TOL)
        assert_close(to_f64(dW1[e][:, icols + I]), uc, "skewed f32 dW1[%d] up" % e, rtol=TOL, atol=TOL)
        assert_close(to_f64(dW2[e][icols]), dr, "skewed f32 dW2[%d]" % e, rtol=TOL, atol=TOL)
