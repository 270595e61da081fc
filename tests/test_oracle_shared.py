"""Pins of the oracle's shared expert (RFC 6.1: a shared expert whose output joins the routed
ones at the Combine; reading: weight 1 for every token, added after the K routed terms).

1. With the shared intermediate size equal to I, the shared expert is exactly an extra routed
   expert E that every token selects last with weight 1: the oracle with shared weights must
   give bit-identical values to the routed oracle on that extended problem (both modes).
2. With a different intermediate size, PURE mode equals torch float64 autograd of the unfused
   chain (library routines, not the oracle's code).
"""

import numpy as np
import pytest
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16


def problem(T, H, I, Is, E, K, seed):
    rng = np.random.default_rng(seed)
    p = dict(
        x=round_bf16(rng.standard_normal((T, H))),
        up_proj_weight=round_bf16(rng.standard_normal((E, H, 2 * I)) / np.sqrt(H)),
        down_proj_weight=round_bf16(rng.standard_normal((E, I, H)) / np.sqrt(I)),
        dY=round_bf16(rng.standard_normal((T, H))),
        topk_ids=np.array([rng.choice(E, K, replace=False) for _ in range(T)]),
    )
    z = rng.standard_normal((T, K))
    p["topk_weights"] = (np.exp(z) / np.exp(z).sum(1, keepdims=True)).astype(np.float32)
    ws1 = round_bf16(rng.standard_normal((H, 2 * Is)) / np.sqrt(H))
    ws2 = round_bf16(rng.standard_normal((Is, H)) / np.sqrt(Is))
    return p, ws1, ws2


@pytest.mark.parametrize("mode", ["faithful", "pure"])
def test_shared_expert_is_an_extra_routed_expert(mode):
    T, H, I, E, K = 48, 64, 32, 4, 2
    p, ws1, ws2 = problem(T, H, I, I, E, K, 3)
    m = MoEFFN(**p, mode=mode, shared_up_proj_weight=ws1, shared_down_proj_weight=ws2)
    ext = dict(p)
    ext["up_proj_weight"] = np.concatenate([p["up_proj_weight"], ws1[None]], 0)
    ext["down_proj_weight"] = np.concatenate([p["down_proj_weight"], ws2[None]], 0)
    ext["topk_ids"] = np.concatenate([p["topk_ids"], np.full((T, 1), E)], 1)
    ext["topk_weights"] = np.concatenate([p["topk_weights"], np.ones((T, 1), np.float32)], 1)
    r = MoEFFN(**ext, mode=mode)
    assert np.array_equal(m.forward(), r.forward())
    (dx, dw, dW1, dW2) = m.backward()
    (rdx, rdw, rdW1, rdW2) = r.backward()
    assert np.array_equal(dx, rdx)
    assert np.array_equal(dw, rdw[:, :K])
    assert np.array_equal(dW1, rdW1[:E]) and np.array_equal(dW2, rdW2[:E])
    (ds1, ds2), _ = m.shared_backward_dev()
    assert np.array_equal(ds1, rdW1[E]) and np.array_equal(ds2, rdW2[E])


def test_shared_expert_pure_matches_torch_autograd():
    T, H, I, Is, E, K = 20, 32, 16, 48, 3, 2
    p, ws1, ws2 = problem(T, H, I, Is, E, K, 4)
    m = MoEFFN(**p, mode="pure", shared_up_proj_weight=ws1, shared_down_proj_weight=ws2)
    f = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)  # noqa: E731
    x, W1, W2, w, S1, S2 = f(p["x"]), f(p["up_proj_weight"]), f(p["down_proj_weight"]), f(p["topk_weights"]), \
        f(ws1), f(ws2)

    def ffn(xr, a1, a2, n):
        h = xr @ a1
        return (torch.nn.functional.silu(h[:, :n]) * h[:, n:]) @ a2

    ids = torch.tensor(p["topk_ids"])
    y = ffn(x, S1, S2, Is)
    for k in range(K):
        parts = [ffn(x[t:t + 1], W1[ids[t, k]], W2[ids[t, k]], I) for t in range(T)]
        y = y + w[:, k:k + 1] * torch.cat(parts, 0)
    y.backward(torch.tensor(p["dY"]))
    assert np.allclose(m.forward(out_dtype="f32"), y.detach().numpy(), rtol=1e-12, atol=1e-12)
    dx, dw, dW1, dW2 = m.backward(out_dtype="f32")
    (ds1, ds2), _ = m.shared_backward_dev(out_dtype="f32")
    for got, ref in ((dx, x.grad), (dw, w.grad), (dW1, W1.grad), (dW2, W2.grad), (ds1, S1.grad), (ds2, S2.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-11, atol=1e-11)
