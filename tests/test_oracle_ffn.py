"""Pins of the oracle's forward and backward.

Each check ties the oracle to something other than itself:
* torch float64 ops (a dense SwiGLU FFN, a dense-masked mixture, autograd of an
  unfused chain written with torch index/matmul ops);
* central finite differences of <dY, y>;
* identities that hold exactly in real arithmetic (degree-1 homogeneity);
* closed forms of tiny cases worked by hand.
"""

import math

import numpy as np
import pytest
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16



def problem(T, H, I, E, K, seed, dup=False, empty=None, bf16=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W1 = rng.standard_normal((E, H, 2 * I)) / np.sqrt(H)
    W2 = rng.standard_normal((E, I, H)) / np.sqrt(I)
    dY = rng.standard_normal((T, H))
    allowed = [e for e in range(E) if e != empty]
    ids = np.array([rng.choice(allowed, size=K, replace=dup) for _ in range(T)])
    z = rng.standard_normal((T, K))
    w = (np.exp(z) / np.exp(z).sum(1, keepdims=True)).astype(np.float32)
    if bf16:
        x, W1, W2, dY = (round_bf16(a) for a in (x, W1, W2, dY))
    return dict(x=x, topk_ids=ids, topk_weights=w, up_proj_weight=W1, down_proj_weight=W2, dY=dY)


def dense_ffn(x, W1e, W2e):
    I = W2e.shape[0]
    h = x @ W1e
    return (torch.nn.functional.silu(h[:, :I]) * h[:, I:]) @ W2e


def torch_chain(p, requires_grad=False):
    """Unfused reference chain in torch float64: permute, per-expert FFN, weighted un-permute."""
    x = torch.tensor(p["x"], dtype=torch.float64, requires_grad=requires_grad)
    W1 = torch.tensor(p["up_proj_weight"], dtype=torch.float64, requires_grad=requires_grad)
    W2 = torch.tensor(p["down_proj_weight"], dtype=torch.float64, requires_grad=requires_grad)
    w = torch.tensor(p["topk_weights"].astype(np.float64), requires_grad=requires_grad)
    ids = torch.tensor(p["topk_ids"], dtype=torch.int64)
    T, K = ids.shape
    E = W1.shape[0]
    flat = ids.reshape(-1)
    order = torch.argsort(flat, stable=True)
    tok = order // K
    xs = x.index_select(0, tok)
    counts = torch.bincount(flat, minlength=E).tolist()
    outs, start = [], 0
    for e in range(E):
        outs.append(dense_ffn(xs[start:start + counts[e]], W1[e], W2[e]))
        start += counts[e]
    o = torch.cat(outs)
    y = torch.zeros(T, x.shape[1], dtype=torch.float64).index_add(0, tok, o * w.reshape(-1)[order][:, None])
    return y, (x, W1, W2, w)


def test_k1_unit_weight_is_dense_ffn():
    p = problem(9, 16, 8, 1, 1, 0, bf16=False)
    p["topk_weights"][:] = 1.0
    y = MoEFFN(**p, mode="pure").forward()
    ref = dense_ffn(torch.tensor(p["x"]), torch.tensor(p["up_proj_weight"][0]),
                    torch.tensor(p["down_proj_weight"][0])).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dup", [False, True])
def test_forward_matches_dense_masked_mixture(dup):
    T, H, I, E, K = 11, 16, 8, 5, 3
    p = problem(T, H, I, E, K, 1, dup=dup, empty=2)
    y = MoEFFN(**p, mode="pure").forward()
    # y_t = sum_e c[t,e] FFN_e(x_t), c[t,e] = sum_k w[t,k] [ids[t,k] == e]; no permutation code
    c = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            c[t, p["topk_ids"][t, k]] += p["topk_weights"][t, k]
    x = torch.tensor(p["x"])
    ref = sum(torch.tensor(c[:, e:e + 1]) * dense_ffn(x, torch.tensor(p["up_proj_weight"][e]),
                                                       torch.tensor(p["down_proj_weight"][e]))
              for e in range(E)).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_one_hot_weights_select_one_slot():
    p = problem(6, 16, 8, 4, 3, 2)
    p["topk_weights"][:] = 0.0
    p["topk_weights"][:, 1] = 1.0
    y = MoEFFN(**p, mode="pure").forward()
    for t in range(6):
        e = p["topk_ids"][t, 1]
        ref = dense_ffn(torch.tensor(p["x"][t:t + 1]), torch.tensor(p["up_proj_weight"][e]),
                        torch.tensor(p["down_proj_weight"][e])).numpy()[0]
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12)


def test_token_reorder_is_equivariant():
    p = problem(10, 16, 8, 4, 2, 3)
    perm = np.random.default_rng(0).permutation(10)
    q = dict(p)
    for k in ("x", "topk_ids", "topk_weights", "dY"):
        q[k] = p[k][perm]
    for mode in ("pure", "faithful"):
        assert np.array_equal(MoEFFN(**p, mode=mode).forward()[perm], MoEFFN(**q, mode=mode).forward())


def test_faithful_rounds_at_stored_points_and_stays_near_pure():
    p = problem(12, 32, 16, 4, 2, 4)
    f = MoEFFN(**p, mode="faithful")
    h, a, o = f.slot_intermediates(np.arange(24))
    for v in (h, a, o):
        assert np.array_equal(round_bf16(v), v)
    yf = f.forward()
    assert np.array_equal(round_bf16(yf), yf)
    yp = MoEFFN(**p, mode="pure").forward()
    assert np.abs(yf - yp).max() <= 0.03 * np.abs(yp).max()


def test_closed_form_faithful_tie_case():
    """H=2, I=1, one expert, one slot; values worked by hand from the definition.

    x = [1, 2^-8], up_proj_weight = [[1, 1], [1, 0]] (gate column, up column),
    down_proj_weight = [[1, 2]], w = 1, dY = [1, 0].
    g = 1 + 2^-8 is a bf16 tie and rounds (R1) to the even neighbour 1; u = 1;
    a = bf16(sigmoid(1)) = 187/256 (sigmoid(1) * 256 = 187.15); o = [a, 2a]; y = o.
    Without R1, silu(1 + 2^-8) * 256 = 188.08 would give 188/256 instead.
    Backward: G = 1, dw = a, dg = bf16(s (1 + (1 - s))) with s = sigmoid(1)
    (* 256 = 237.48 -> 237/256), du = bf16(s) = 187/256;
    dXp = [dg + du, dg] (both exact in bf16), dx = dXp.
    """
    f = MoEFFN(np.array([[1.0, 2.0 ** -8]]), np.array([[0]]), np.array([[1.0]], np.float32),
               np.array([[[1.0, 1.0], [1.0, 0.0]]]), np.array([[[1.0, 2.0]]]),
               dY=np.array([[1.0, 0.0]]), mode="faithful")
    a = 187 / 256
    assert np.array_equal(f.forward(), np.array([[a, 2 * a]]))
    dx, dw = f.backward_tokens()
    dg, du = 237 / 256, 187 / 256
    assert np.array_equal(dx, np.array([[dg + du, dg]]))
    assert dw[0, 0] == a


def test_closed_form_pure_two_experts():
    """x = [2]; expert 0: gate 1, up 1, down 1; expert 1: gate 0, up 3, down 5; w = [1/4, 3/4].

    Slot 0: g = u = 2, a = 4 s2 with s2 = sigmoid(2); slot 1: g = 0 so a = 0.
    y = a / 4 = s2.  With dY = 1: dw = [4 s2, 0]; slot 0: dA = 1/4,
    dg = (1/4) 2 s2 (1 + 2 (1 - s2)), du = (1/4) 2 s2; slot 1: dA = 15/4, dg = 15/4 * 6 / 2,
    du = 0, and its input gradient is dg * 0 + du * 3 = 0.  dx = dg0 + du0.
    """
    f = MoEFFN(np.array([[2.0]]), np.array([[0, 1]]), np.array([[0.25, 0.75]], np.float32),
               np.array([[[1.0, 1.0]], [[0.0, 3.0]]]), np.array([[[1.0]], [[5.0]]]),
               dY=np.array([[1.0]]), mode="pure")
    s2 = 1.0 / (1.0 + math.exp(-2.0))
    assert np.allclose(f.forward(), [[s2]], rtol=1e-15, atol=0)
    dx, dw = f.backward_tokens()
    assert np.allclose(dw, [[4 * s2, 0.0]], rtol=1e-15, atol=0)
    dg0 = 0.25 * 2 * s2 * (1 + 2 * (1 - s2))
    du0 = 0.25 * 2 * s2
    assert np.allclose(dx, [[dg0 + du0]], rtol=1e-15, atol=0)
    _, dw1u, dw2r = f.weight_grads_expert(1)
    dw1g, _, _ = f.weight_grads_expert(1)
    assert np.allclose(dw1g, [[2 * 15 / 4 * 6 / 2]], rtol=1e-15)   # x * dg of slot 1
    assert np.allclose(dw2r, [[0.0]])                                 # a = 0 on slot 1


# ----------------------------------------------------------------------------- backward

def test_backward_matches_torch_autograd_of_unfused_chain():
    p = problem(14, 32, 16, 5, 3, 5, dup=True, empty=1)
    dx, dw, dW1, dW2 = MoEFFN(**p, mode="pure").backward()
    y, (x, W1, W2, w) = torch_chain(p, requires_grad=True)
    y.backward(torch.tensor(p["dY"]))
    assert np.allclose(dx, x.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dW1, W1.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dW2, W2.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dw, w.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.all(dW1[1] == 0) and np.all(dW2[1] == 0)


def test_backward_matches_central_finite_differences():
    p = problem(6, 16, 8, 3, 2, 6, dup=True, empty=2, bf16=False)
    # force one duplicate id inside a token
    p["topk_ids"][0] = [1, 1]
    base = MoEFFN(**p, mode="pure")
    dx, dw, dW1, dW2 = base.backward()
    dY = p["dY"]

    def loss(q):
        return float(np.sum(dY * MoEFFN(**q, mode="pure").forward()))

    rng = np.random.default_rng(0)
    for name, grad in (("x", dx), ("up_proj_weight", dW1), ("down_proj_weight", dW2), ("topk_weights", dw)):
        arr = p[name]
        idxs = [np.unravel_index(i, arr.shape) for i in rng.choice(arr.size, size=min(arr.size, 40), replace=False)]
        # topk_weights are float32 inputs: step by 2^-10, which float32 holds exactly
        # (y is linear in them, so the central difference is exact up to rounding)
        eps = 2.0 ** -10 if name == "topk_weights" else 1e-6
        for idx in idxs:
            q = {k: (v.astype(np.float64).copy() if isinstance(v, np.ndarray) and k != "topk_ids" else v)
                 for k, v in p.items()}
            q[name][idx] += eps
            lp = loss(q)
            q[name][idx] -= 2 * eps
            lm = loss(q)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_backward_homogeneity_identities():
    # y is degree-1 homogeneous in w, in W2 and in the up half of W1
    p = problem(10, 32, 16, 4, 2, 7)
    m = MoEFFN(**p, mode="pure")
    y = m.forward()
    dx, dw, dW1, dW2 = m.backward()
    I = 16
    ref = np.sum(p["dY"] * y)
    assert np.isclose(np.sum(dw * p["topk_weights"]), ref, rtol=1e-10)
    assert np.isclose(np.sum(dW2 * p["down_proj_weight"]), ref, rtol=1e-10)
    assert np.isclose(np.sum(dW1[:, :, I:] * p["up_proj_weight"][:, :, I:]), ref, rtol=1e-10)


def test_backward_is_linear_in_dy():
    p = problem(8, 16, 8, 3, 2, 8)
    q = dict(p, dY=np.random.default_rng(1).standard_normal(p["dY"].shape))
    s = dict(p, dY=p["dY"] + q["dY"])
    g1, g2, g3 = (MoEFFN(**z, mode="pure").backward() for z in (p, q, s))
    for a, b, c in zip(g1, g2, g3):
        assert np.allclose(a + b, c, rtol=1e-11, atol=1e-12)


def test_samplers_agree_with_full_backward():
    p = problem(20, 32, 16, 4, 3, 9, empty=3)
    for mode in ("pure", "faithful"):
        m = MoEFFN(**p, mode=mode)
        dx, dw, dW1, dW2 = m.backward()
        toks = np.array([0, 7, 19])
        sdx, sdw = m.backward_tokens(toks)
        assert np.array_equal(sdx, dx[toks]) and np.array_equal(sdw, dw[toks])
        icols = np.array([1, 5, 15])
        for e in range(4):
            g, u, r = m.weight_grads_expert(e, icols)
            assert np.allclose(g, dW1[e][:, icols], rtol=1e-14, atol=0)
            assert np.allclose(u, dW1[e][:, icols + 16], rtol=1e-14, atol=0)
            assert np.allclose(r, dW2[e][icols], rtol=1e-14, atol=0)
        assert np.all(dW1[3] == 0) and np.all(dW2[3] == 0)
        assert np.allclose(m.forward(toks), m.forward()[toks], rtol=0, atol=0)


def test_faithful_backward_rounds_and_stays_near_pure():
    p = problem(16, 32, 16, 4, 2, 10)
    f = MoEFFN(**p, mode="faithful").backward()
    q = MoEFFN(**p, mode="pure").backward()
    for a in (f[0], f[2], f[3]):
        assert np.array_equal(round_bf16(a), a)
    for a, b in zip(f, q):
        assert np.abs(a - b).max() <= 0.05 * np.abs(b).max()
