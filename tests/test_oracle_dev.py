"""Pins of the oracle's admissible-deviation bound (FAITHFUL mode).

A second implementation of the same bfloat16 pipeline, written with torch
float32 CPU ops and grouped by expert (so every sum runs in another order and
precision than the oracle's float64 per-token loop), must land within the
oracle's ``dev`` bound on every element, with no other tolerance.  Where the
two differ, they differ because a rounding decision was open; the bound has to
cover exactly that.
"""

import numpy as np
import pytest
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16


def bf(t):
    return t.to(torch.bfloat16).to(torch.float32)


def f32_pipeline(p, up=None):
    """Independent float32 pipeline: permute by expert, grouped matmuls, bf16 at R1..R9.

    ``up(X, e)`` replaces the up-projection X . W1[e] (float32 result, before R1)."""
    f = lambda a: torch.tensor(np.asarray(a), dtype=torch.float32)  # noqa: E731
    x, W1, W2, dY = f(p["x"]), f(p["up_proj_weight"]), f(p["down_proj_weight"]), f(p["dY"])
    w = f(p["topk_weights"])
    ids = torch.tensor(p["topk_ids"], dtype=torch.int64)
    T, K = ids.shape
    E, H, I2 = W1.shape
    I = I2 // 2
    flat = ids.reshape(-1)
    o = torch.zeros(T * K, H)
    dxp = torch.zeros(T * K, H)
    dw = torch.zeros(T * K)
    dW1 = torch.zeros(E, H, I2)
    dW2 = torch.zeros(E, I, H)
    for e in range(E):
        slots = torch.nonzero(flat == e).reshape(-1)
        if slots.numel() == 0:
            continue
        tok = slots // K
        ws = w.reshape(-1)[slots][:, None]
        X = x[tok]
        h = bf(X @ W1[e] if up is None else up(X, e))
        g, u = h[:, :I], h[:, I:]
        s = torch.sigmoid(g)
        a = bf(g * s * u)
        aw = bf(ws * a)
        o[slots] = bf(a @ W2[e])
        D = dY[tok]
        G = D @ W2[e].T
        dw[slots] = (G * a).sum(1)
        dA = ws * G
        dg = bf(dA * u * s * (1 + g * (1 - s)))
        du = bf(dA * g * s)
        dH = torch.cat([dg, du], 1)
        dxp[slots] = bf(dH @ W1[e].T)
        dW1[e] = bf(X.T @ dH)
        dW2[e] = bf(aw.T @ D)
    o = o.reshape(T, K, H)
    y = bf((w[:, :, None] * o).sum(1))
    dx = bf(dxp.reshape(T, K, H).sum(1))
    return [v.double().numpy() for v in (y, dx, dw.reshape(T, K), dW1, dW2)]


def problem(T, H, I, E, K, seed):
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
    return p


@pytest.mark.parametrize("T,H,I,E,K,seed", [(256, 512, 256, 4, 2, 0), (300, 256, 128, 6, 3, 1)])
def test_float32_pipeline_within_dev(T, H, I, E, K, seed):
    p = problem(T, H, I, E, K, seed)
    m = MoEFFN(**p, mode="faithful")
    y, yd = m.forward_dev()
    (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d) = m.backward_dev()
    got = f32_pipeline(p)
    n_diff = 0
    for name, g, r, d in zip(("y", "dx", "dw", "dW1", "dW2"), got, (y, dx, dw, dW1, dW2), (yd, dxd, dwd, dW1d, dW2d)):
        err = np.abs(g - r)
        bad = err > d
        assert not bad.any(), "%s: %d entries beyond dev; worst %r" % (name, bad.sum(), (err - d).max())
        if name != "dw":
            n_diff += int((g != r).sum())
    # the check is not vacuous: some rounding decisions did come out differently
    assert n_diff > 0


def test_dev_is_zero_in_pure_mode_and_mostly_zero_in_faithful():
    p = problem(64, 128, 64, 3, 2, 2)
    _, d = MoEFFN(**p, mode="pure").forward_dev()
    assert not d.any()
    y, d = MoEFFN(**p, mode="faithful").forward_dev()
    assert (d == 0).mean() > 0.75
    # a few bf16 ulps of the value, or a small absolute amount next to zero (cancellation)
    ulp = np.spacing(np.abs(y).astype(np.float32)).astype(np.float64) * 2 ** 16
    assert np.all(d <= 4 * ulp + 1e-3 * np.abs(y).max())


def test_dev_flags_a_rounding_tie():
    """g = 1 + 2^-8 is a bf16 tie: a float32 evaluation may land on either side."""
    m = MoEFFN(np.array([[1.0, 2.0 ** -8]]), np.array([[0]]), np.array([[1.0]], np.float32),
               np.array([[[1.0, 1.0], [1.0, 0.0]]]), np.array([[[1.0, 2.0]]]), mode="faithful")
    (g, u, a), (gd, ud, ad) = m.hidden_dev(0, m.x)
    assert g[0, 0] == 1.0 and gd[0, 0] == 2.0 ** -7      # the other neighbour, 1 + 2^-7, is admissible
    assert ud[0, 0] == 0.0                               # u = 1 exactly: no doubt
    assert ad[0, 0] > 0                                  # the doubt on g reaches a


def _e4m3_rows(a):
    """Per-row dynamic E4M3 quantisation with torch's float8 cast: (values, descale), float32 scale math."""
    amax = a.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, torch.tensor(448.0) / amax, torch.ones_like(amax))
    q = (a * scale).to(torch.float8_e4m3fn).to(torch.float64)
    return q, (1.0 / scale).to(torch.float64)


def _fp8_instruction_sum(qa, qb, group=8, keep_bits=13):
    """A model of an FP8 matrix instruction's sum: the products of each group of ``group``
    consecutive k are truncated toward zero to ``keep_bits`` bits below the group's largest
    product, summed, and the group sums added into a float32 accumulator."""
    n, H = qa.shape
    t = qa[:, :, None] * qb[None, :, :]                          # [n, H, N], exact
    t = t.reshape(n, H // group, group, -1)
    m = np.abs(t).max(axis=2, keepdims=True)
    quantum = np.where(m > 0, np.exp2(np.floor(np.log2(np.where(m > 0, m, 1.0))) - keep_bits), 1.0)
    gs = (np.trunc(t / quantum) * quantum).sum(axis=2)           # [n, H/group, N]
    acc = np.zeros((n, t.shape[-1]), np.float32)
    for j in range(gs.shape[1]):
        acc = (acc + gs[:, j].astype(np.float32)).astype(np.float32)
    return acc


@pytest.mark.parametrize("T,H,I,E,K,seed", [(128, 256, 64, 4, 2, 3), (96, 512, 64, 3, 3, 4)])
def test_fp8_instruction_model_within_dev(T, H, I, E, K, seed):
    """The FP8 variant's R1 deviation covers a matrix instruction that keeps only ~13 bits per group."""
    p = problem(T, H, I, E, K, seed)
    p["x"][::7] *= 16.0                                          # outlier rows
    W1 = torch.tensor(p["up_proj_weight"], dtype=torch.float32)
    wq, wds = zip(*[_e4m3_rows(W1[e].T) for e in range(E)])     # per-column quantisation

    def up(X, e):
        xq, xds = _e4m3_rows(X)
        acc = _fp8_instruction_sum(xq.numpy(), wq[e].T.numpy())
        return (torch.tensor(acc) * xds.float()) * wds[e].float().reshape(1, -1)

    m = MoEFFN(**p, mode="faithful", gmm1="fp8")
    y, yd = m.forward_dev()
    (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d) = m.backward_dev()
    got = f32_pipeline(p, up)
    for name, g, r, d in zip(("y", "dx", "dw", "dW1", "dW2"), got, (y, dx, dw, dW1, dW2), (yd, dxd, dwd, dW1d, dW2d)):
        bad = np.abs(g - r) > d
        assert not bad.any(), "%s: %d entries beyond dev" % (name, bad.sum())
