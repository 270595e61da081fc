"""FP8 backward on the GPU (HMM_FLAG_FP8_BACKWARD: act_grad and input_grad on E4M3
with per-row dynamic scales) against the oracle's FP8-backward mode.

Every output is compared element by element under the oracle's deviation bound.
That bound is wide for dx, because dH is an intermediate whose open bf16 decisions
can move an E4M3 code by a whole step.  So the tests also require nearly every
element of every output within the plain bar (1e-2 + 1e-2 |ref|): the bound may
only absorb what it is there for.
"""

import numpy as np
import pytest

from _util import ATOL, RTOL, announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from test_gpu_parity import _sample_full, run_gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict(T=128, H=128, I=64, E=4, K=2)),
    ("ragged", dict(T=300, H=256, I=192, E=6, K=3, routing="uniform")),
    ("zipf", dict(T=411, H=384, I=128, E=16, K=4, routing="zipf", zipf_s=1.2, n_empty=5)),
    ("outliers", dict(T=520, H=256, I=320, E=3, K=2, routing="hot", outlier_frac=0.02, outlier_scale=30.0)),
    # many experts: on 64x64 tiles the launches spread the real tiles over the XCDs
    ("e1024", dict(T=512, H=128, I=64, E=1024, K=8, routing="zipf", zipf_s=0.6, n_empty=200)),
]
PLAIN_SHARE = 0.01   # at most this share of an output's elements outside the plain bar


def _check(got, ref, dev, name):
    assert_close(got, ref, name, dev)
    outside = np.abs(np.asarray(got, np.float64) - ref) > ATOL + RTOL * np.abs(ref)
    assert outside.mean() <= PLAIN_SHARE, "%s: %.3f%% of entries outside the plain bar" % (name, 100 * outside.mean())


@pytest.mark.parametrize("gmm1", ["bf16", "fp8"])
@pytest.mark.parametrize("tiles", ["large", "narrow"])
@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_fp8_backward_parity(name, over, tiles, gmm1):
    spec = synth.spec_with("tiny", **over)
    inp = synth.make_inputs(spec, seed=31)
    announce("fp8 backward %s %s tiles=%s up-projection %s" % (name, {k: spec[k] for k in "THIEK"}, tiles, gmm1))
    g = gpu_inputs(inp, "cuda")
    y, saved, dx, dW1, dW2, dw = run_gpu(g, tiles, gmm1=gmm1, fp8_backward=True)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1=gmm1, bwd="fp8")
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    _check(to_f64(dx), rdx, ddx, name + " dx")
    _check(to_f64(dw), rdw, ddw, name + " d_topk_weights")
    _check(to_f64(dW1), rdW1, ddW1, name + " d_up_proj_weight")
    _check(to_f64(dW2), rdW2, ddW2, name + " d_down_proj_weight")
    counts = np.bincount(inp["topk_ids"].reshape(-1), minlength=spec["E"])
    for e in np.flatnonzero(counts == 0):
        assert not to_f64(dW1[e]).any() and not to_f64(dW2[e]).any()


def test_fp8_backward_with_shared_expert():
    """The routed products on E4M3, the shared expert's in bf16 (as the oracle reads it)."""
    from mixture_experts_ffn_int32_amd import backward_from_saved, forward_with_saved
    spec = synth.spec_with("tiny", T=300, H=256, I=192, E=6, K=3, routing="uniform", shared_I=128)
    inp = synth.make_inputs(spec, seed=32)
    announce("fp8 backward with a shared expert")
    g = gpu_inputs(inp, "cuda")
    sh = dict(shared_up_proj_weight=g["shared_up_proj_weight"], shared_down_proj_weight=g["shared_down_proj_weight"])
    y, saved = forward_with_saved(g["x"], g["topk_ids"], g["topk_weights"], g["up_proj_weight"],
                                  g["down_proj_weight"], tiles="large", **sh)
    dx, dW1, dW2, dw, dWs1, dWs2 = backward_from_saved(g["dY"], g["x"], g["topk_ids"], g["topk_weights"],
                                                       g["up_proj_weight"], g["down_proj_weight"], saved,
                                                       tiles="large", fp8_backward=True, **sh)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", bwd="fp8")
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    (rs1, rs2), (ds1, ds2) = o.shared_backward_dev()
    _check(to_f64(dx), rdx, ddx, "dx")
    _check(to_f64(dw), rdw, ddw, "d_topk_weights")
    _check(to_f64(dW1), rdW1, ddW1, "d_up_proj_weight")
    _check(to_f64(dW2), rdW2, ddW2, "d_down_proj_weight")
    _check(to_f64(dWs1), rs1, ds1, "d_shared_up_proj_weight")
    _check(to_f64(dWs2), rs2, ds2, "d_shared_down_proj_weight")


def test_fp8_backward_differs_from_bf16_and_autograd_matches_raw():
    import torch
    from mixture_experts_ffn_int32_amd import hyper_mega_moe
    spec = synth.spec_with("tiny", T=256, H=256, I=128, E=4, K=2)
    g = gpu_inputs(synth.make_inputs(spec, seed=33), "cuda")
    announce("fp8 backward under autograd")
    x = g["x"].clone().requires_grad_(True)
    w = g["topk_weights"].clone().requires_grad_(True)
    W1 = g["up_proj_weight"].clone().requires_grad_(True)
    W2 = g["down_proj_weight"].clone().requires_grad_(True)
    y = hyper_mega_moe(x, g["topk_ids"], w, W1, W2, fp8_backward=True)
    y.backward(g["dY"])
    _, _, dx, dW1, dW2, dw = run_gpu(g, fp8_backward=True)
    _, _, dx16, *_ = run_gpu(g)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, dx) and torch.equal(W1.grad, dW1) and torch.equal(W2.grad, dW2)
    assert torch.equal(w.grad, dw)
    assert not torch.equal(dx, dx16)
    rel = ((dx.float() - dx16.float()).norm() / dx16.float().norm()).item()
    assert rel < 0.1, rel


@pytest.mark.slow
def test_full_size_fp8_backward_sampled():
    """The FP8 workload (T=16384, H=4096, I=1536, E=64, K=6) with the FP8 backward."""
    _sample_full("fp8bwd", n_tok=4)
