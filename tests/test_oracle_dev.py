"""Pins of the oracle's admissible-deviation bound (FAITHFUL mode), from both sides.

From below: a second implementation of the same bfloat16 pipeline, written with
torch float32 CPU ops and grouped by expert (so every sum runs in another order
and precision than the oracle's float64 per-token loop), must land within the
oracle's ``dev`` bound on every element, with no other tolerance.  Where the
two differ, they differ because a rounding decision was open; the bound has to
cover exactly that.  The quantised variants run the same pipeline with a model
of the FP8 matrix instruction in the up-projection.

From above: at a hidden size of 2048, dev measured against the stated
tolerance (1e-2 + 1e-2 |ref|) stays below per-output limits on its median and
99th percentile, so the bound cannot grow into a wide extra tolerance.
"""

import numpy as np
import pytest
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16


def bf(t):
    return t.to(torch.bfloat16).to(torch.float32)


def f32_pipeline(p, up=None, ag=None, ig=None):
    """Independent float32 pipeline: permute by expert, grouped matmuls, bf16 at R1..R9.

    ``up(X, e)`` replaces the up-projection X . W1[e] (float32 result, before R1);
    ``ag(D, e)`` the act_grad product D . W2[e]^T and ``ig(dH, e)`` the input_grad
    product dH . W1[e]^T (float32 results, before their rounding)."""
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
        G = D @ W2[e].T if ag is None else ag(D, e)
        dw[slots] = (G * a).sum(1)
        dA = ws * G
        dg = bf(dA * u * s * (1 + g * (1 - s)))
        du = bf(dA * g * s)
        dH = torch.cat([dg, du], 1)
        dxp[slots] = bf(dH @ W1[e].T if ig is None else ig(dH, e))
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


def _frexp_exp(a):
    """floor(log2 a) for a > 0 (exact, via frexp)."""
    return torch.frexp(a)[1].to(torch.float64) - 1


def _mx_dequant_rows(a):
    """MX quantisation of the rows of ``a`` [n, H] (blocks of 32, exponent floor(log2 max) - 8,
    clamped to [-127, 127], -127 for a zero block; saturating E4M3 cast), returned dequantised."""
    n, H = a.shape
    b = a.to(torch.float64).reshape(n, H // 32, 32)
    amax = b.abs().amax(-1, keepdim=True)
    e = torch.where(amax > 0, _frexp_exp(torch.where(amax > 0, amax, torch.ones_like(amax))) - 8,
                    torch.full_like(amax, -127.0)).clamp(-127, 127)
    q = (b / torch.exp2(e)).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * torch.exp2(e)).reshape(n, H)


def _fp8_model_up(p, gmm1):
    """up(X, e) of f32_pipeline with the FP8 instruction model, for gmm1 = fp8 | mx | group."""
    W1 = torch.tensor(p["up_proj_weight"], dtype=torch.float32)
    E = W1.shape[0]
    if gmm1 == "fp8":
        wq, wds = zip(*[_e4m3_rows(W1[e].T) for e in range(E)])   # per-column quantisation

        def up(X, e):
            xq, xds = _e4m3_rows(X)
            acc = _fp8_instruction_sum(xq.numpy(), wq[e].T.numpy())
            return (torch.tensor(acc) * xds.float()) * wds[e].float().reshape(1, -1)
    elif gmm1 == "mx":
        wd = [_mx_dequant_rows(W1[e].T).T.numpy() for e in range(E)]   # blocks of 32 rows per column

        def up(X, e):
            return torch.tensor(_fp8_instruction_sum(_mx_dequant_rows(X).numpy(), wd[e]))
    else:
        G = 128
        H = W1.shape[1]
        wg = [_e4m3_rows(W1[e].T.reshape(-1, H // G, G)) for e in range(E)]   # [2I, H/G, G] codes, [2I, H/G, 1]

        def up(X, e):
            n = X.shape[0]
            xq, xds = _e4m3_rows(X.reshape(n, H // G, G))
            wq, wds = wg[e]
            acc = np.zeros((n, wq.shape[0]), np.float32)
            for g in range(H // G):           # group sums scaled and added in float32, in group order
                s = _fp8_instruction_sum(xq[:, g].numpy(), wq[:, g].T.numpy())
                sc = (xds[:, g].float() * wds[:, g].float().reshape(1, -1)).numpy()
                acc = (acc + (s * sc).astype(np.float32)).astype(np.float32)
            return torch.tensor(acc)
    return up


@pytest.mark.parametrize("gmm1", ["fp8", "mx", "group"])
def test_fp8_instruction_model_within_dev_at_h2048(gmm1):
    """At a hidden size of 2048 (with outlier rows), the float32 pipeline with the FP8
    instruction model stays within dev in every quantised variant, and does differ."""
    p = problem(32, 2048, 768, 8, 2, 5)
    p["x"][::7] *= 16.0
    m = MoEFFN(**p, mode="faithful", gmm1=gmm1)
    y, yd = m.forward_dev()
    (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d) = m.backward_dev()
    got = f32_pipeline(p, _fp8_model_up(p, gmm1))
    n_diff = 0
    for name, g, r, d in zip(("y", "dx", "dw", "dW1", "dW2"), got, (y, dx, dw, dW1, dW2), (yd, dxd, dwd, dW1d, dW2d)):
        bad = np.abs(g - r) > d
        assert not bad.any(), "%s: %d entries beyond dev" % (name, bad.sum())
        if name != "dw":
            n_diff += int((g != r).sum())
    assert n_diff > 0


# Upper limits of dev / (1e-2 + 1e-2 |ref|): (median, 99th percentile) per output.
# Measured at T=32, H=2048, I=768, E=8, K=2, seed 7 (in brackets):
#   bf16: y 0.15 / 0.49, dx 0.31 / 0.74, dW1 0 / 0.42, dW2 0 / 0.34, d_topk_weights 0.23 / 6.0;
#   fp8, mx, group: y 0.77 / 1.5, dx 0.86 / 1.5, dW1 0.09 / 1.1, dW2 0.16 / 1.4,
#   d_topk_weights 1.5 / 16-41.
# d_topk_weights = sum_i G_i a_i over I terms is the one output whose value is
# routinely far below the size of its terms (|G a| ~ 0.5 each, sums of order 1
# at the 99th percentile): a few open bf16 decisions of a move it by more than
# 1e-2 |ref| there.  The quantised variants' R1 is open on ~13% of h (the FP8
# instruction's accumulation error, ~2^-12 of sqrt(sum t^2)), against ~1% in
# bf16 (float32 accumulation, ~2^-16).
DEV_LIMITS = {
    "bf16": {"y": (0.25, 1.0), "dx": (0.4, 1.0), "dw": (0.35, 8.0), "dW1": (0.05, 1.0), "dW2": (0.05, 1.0)},
    "fp8": {"y": (1.0, 2.0), "dx": (1.0, 2.0), "dw": (2.0, 50.0), "dW1": (0.15, 1.5), "dW2": (0.25, 2.0)},
}
DEV_LIMITS["mx"] = DEV_LIMITS["group"] = DEV_LIMITS["fp8"]
# FP8 backward (act_grad and input_grad on E4M3): dH is an intermediate, and where a bf16
# decision of dH is open its E4M3 code may be the next one (a step of 6-12% of the
# element), so dx's bound widens.  Measured (seed 7): bf16 up-projection dx 2.1 / 8.0,
# d_topk_weights 0.28 / 12, dW1 0.04 / 0.76, dW2 0 / 0.34; FP8 up-projection dx 4.6 / 11,
# d_topk_weights 1.5 / 47, dW1 0.22 / 1.3, dW2 0.16 / 1.4.
DEV_LIMITS["bf16+fp8bwd"] = dict(DEV_LIMITS["bf16"], dx=(2.5, 10.0), dw=(0.35, 15.0), dW1=(0.06, 1.0))
DEV_LIMITS["fp8+fp8bwd"] = dict(DEV_LIMITS["fp8"], dx=(5.0, 13.0), dw=(2.0, 55.0), dW1=(0.3, 1.5))


@pytest.mark.parametrize("gmm1", ["bf16", "fp8", "mx", "group", "bf16+fp8bwd", "fp8+fp8bwd"])
def test_dev_bounded_above_at_h2048(gmm1):
    p = problem(32, 2048, 768, 8, 2, 7)
    up, _, bwd = gmm1.partition("+")
    m = MoEFFN(**p, mode="faithful", gmm1=up, bwd="fp8" if bwd else "bf16")
    y, yd = m.forward_dev()
    (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d) = m.backward_dev()
    for name, r, d in zip(("y", "dx", "dw", "dW1", "dW2"), (y, dx, dw, dW1, dW2), (yd, dxd, dwd, dW1d, dW2d)):
        q = d / (1e-2 + 1e-2 * np.abs(r))
        med, p99 = np.median(q), np.percentile(q, 99)
        lm, lp = DEV_LIMITS[gmm1][name]
        assert med <= lm and p99 <= lp, "%s %s: dev/tol median %.3g (limit %g), p99 %.3g (limit %g)" % (
            gmm1, name, med, lm, p99, lp)


def _fp8_backward_model(p):
    """ag, ig hooks of f32_pipeline for the FP8 backward: per-row E4M3 quantisation (torch
    float32 ops and float8 cast) of dY, dH and the rows of W2[e] and W1[e], the instruction
    model's sums, float32 descales."""
    W1 = torch.tensor(p["up_proj_weight"], dtype=torch.float32)
    W2 = torch.tensor(p["down_proj_weight"], dtype=torch.float32)
    E = W1.shape[0]
    w2r = [_e4m3_rows(W2[e]) for e in range(E)]            # rows i over H
    w1r = [_e4m3_rows(W1[e]) for e in range(E)]            # rows h over 2I

    def prod(A, wr):
        aq, ads = _e4m3_rows(A)
        acc = _fp8_instruction_sum(aq.numpy(), wr[0].T.numpy())
        return (torch.tensor(acc) * ads.float()) * wr[1].float().reshape(1, -1)
    return (lambda D, e: prod(D, w2r[e])), (lambda dH, e: prod(dH, w1r[e]))


@pytest.mark.parametrize("gmm1", ["bf16", "fp8"])
def test_fp8_backward_model_within_dev_at_h2048(gmm1):
    """The FP8 backward (act_grad and input_grad on E4M3) through the float32 pipeline with
    the instruction model stays within dev, with a bf16 or an FP8 up-projection."""
    p = problem(32, 2048, 768, 8, 2, 5)
    p["x"][::7] *= 16.0
    m = MoEFFN(**p, mode="faithful", gmm1=gmm1, bwd="fp8")
    y, yd = m.forward_dev()
    (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d) = m.backward_dev()
    ag, ig = _fp8_backward_model(p)
    got = f32_pipeline(p, _fp8_model_up(p, gmm1) if gmm1 != "bf16" else None, ag, ig)
    n_diff = 0
    for name, g, r, d in zip(("y", "dx", "dw", "dW1", "dW2"), got, (y, dx, dw, dW1, dW2), (yd, dxd, dwd, dW1d, dW2d)):
        bad = np.abs(g - r) > d
        assert not bad.any(), "%s: %d entries beyond dev" % (name, bad.sum())
        if name in ("dx", "dW1"):
            n_diff += int((g != r).sum())
    assert n_diff > 0
