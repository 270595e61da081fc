"""Parity on shapes drawn at random (a fixed seed, so the cases are the same every
run): token counts, widths, expert counts from 1 to 1000, top-k, the three
routings and the three tilings, each case forward and backward against the
oracle's FAITHFUL mode; and the same for the quantised up-projections (per
token, MX, per group) with or without the FP8 backward.  Complements the
hand-picked shapes of test_gpu_parity.py with combinations nobody chose (table
capacities far above or near the real tile counts, counts that do not divide
the XCD count, ...)."""
import numpy as np
import pytest

from _util import announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from test_gpu_parity import run_gpu


def _cases(n, seed=2024, hstep=64):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 128, 257, 1000]))
        K = int(rng.integers(1, min(8, E) + 1))
        over = dict(T=int(rng.integers(1, 1500)), H=int(hstep * rng.integers(1, 512 // hstep + 1)),
                    I=int(64 * rng.integers(1, 7)),
                    E=E, K=K, routing=str(rng.choice(["uniform", "zipf", "hot"] if E > 1 else ["uniform"])))
        if over["routing"] == "zipf":
            over.update(zipf_s=float(rng.uniform(0.5, 1.5)), n_empty=int(rng.integers(0, max(1, E // 4))))
        out.append((over, str(rng.choice(["large", "narrow", "auto"])), int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases(16)
# the FP8 products need H a multiple of 128
Q_CASES = [(over, tiles, seed, mode, seed % 2 == 1)
           for (over, tiles, seed), mode in zip(_cases(8, seed=77, hstep=128), ["fp8", "mx", "group", "fp8"] * 2)]


@pytest.mark.gpu
@pytest.mark.parametrize("over,tiles,seed", CASES, ids=["case%02d" % i for i in range(len(CASES))])
def test_random_shape_parity(over, tiles, seed):
    spec = synth.spec_with("tiny", **over)
    announce("random parity %s routing=%s tiles=%s seed=%d" % ({k: spec[k] for k in "THIEK"}, spec["routing"],
                                                               tiles, seed))
    inp = synth.make_inputs(spec, seed=seed)
    y, saved, dx, dW1, dW2, dw = run_gpu(gpu_inputs(inp, "cuda"), tiles)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, "y", ryd)
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    assert_close(to_f64(dx), rdx, "dx", ddx)
    assert_close(to_f64(dw), rdw, "d_topk_weights", ddw)
    assert_close(to_f64(dW1), rdW1, "d_up_proj_weight", ddW1)
    assert_close(to_f64(dW2), rdW2, "d_down_proj_weight", ddW2)


@pytest.mark.gpu
@pytest.mark.parametrize("over,tiles,seed,gmm1,fp8bwd", Q_CASES, ids=["q%02d" % i for i in range(len(Q_CASES))])
def test_random_shape_parity_quantised(over, tiles, seed, gmm1, fp8bwd):
    spec = synth.spec_with("tiny", **over)
    announce("random parity %s routing=%s tiles=%s gmm1=%s fp8_backward=%s seed=%d"
             % ({k: spec[k] for k in "THIEK"}, spec["routing"], tiles, gmm1, fp8bwd, seed))
    inp = synth.make_inputs(spec, seed=seed)
    y, saved, dx, dW1, dW2, dw = run_gpu(gpu_inputs(inp, "cuda"), tiles, gmm1=gmm1, fp8_backward=fp8bwd)
    o = MoEFFN(**oracle_inputs(inp), mode="faithful", gmm1=gmm1, bwd="fp8" if fp8bwd else "bf16")
    ry, ryd = o.forward_dev()
    assert_close(to_f64(y), ry, "y", ryd)
    (rdx, rdw, rdW1, rdW2), (ddx, ddw, ddW1, ddW2) = o.backward_dev()
    assert_close(to_f64(dx), rdx, "dx", ddx)
    assert_close(to_f64(dw), rdw, "d_topk_weights", ddw)
    assert_close(to_f64(dW1), rdW1, "d_up_proj_weight", ddW1)
    assert_close(to_f64(dW2), rdW2, "d_down_proj_weight", ddW2)
