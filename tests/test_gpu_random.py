"""Parity on shapes drawn at random (a fixed seed, so the cases are the same every
run): token counts, widths, expert counts from 1 to 1000, top-k, the three
routings and the three tilings, each case forward and backward against the
oracle's FAITHFUL mode.  Complements the hand-picked shapes of
test_gpu_parity.py with combinations nobody chose (table capacities far above or
near the real tile counts, counts that do not divide the XCD count, ...)."""
import numpy as np
import pytest

from _util import announce, assert_close, gpu_inputs, oracle_inputs, to_f64
from mixture_experts_ffn_int32_amd import synth
from oracle.moe_ffn import MoEFFN
from test_gpu_parity import run_gpu


def _cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 128, 257, 1000]))
        K = int(rng.integers(1, min(8, E) + 1))
        over = dict(T=int(rng.integers(1, 1500)), H=int(64 * rng.integers(1, 9)), I=int(64 * rng.integers(1, 7)),
                    E=E, K=K, routing=str(rng.choice(["uniform", "zipf", "hot"] if E > 1 else ["uniform"])))
        if over["routing"] == "zipf":
            over.update(zipf_s=float(rng.uniform(0.5, 1.5)), n_empty=int(rng.integers(0, max(1, E // 4))))
        out.append((over, str(rng.choice(["large", "narrow", "auto"])), int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases(16)


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
