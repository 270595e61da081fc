"""Forward and backward of the MoE-FFN expert computation (oracle, float64).

What is computed (HyperMegaMoE RFC sections 2.1, 2.2, 3.1, 4.1, 4.2; usage
guide, "inputs and weights"):

for every token t and every k < K, with e = topk_ids[t, k]:
    [g | u] = x[t] . up_proj_weight[e]          (up_proj_weight is [E, H, 2I];
                                                 the first I columns are the
                                                 gate, the last I the up part)
    a       = silu(g) * u                       (the activation is SwiGLU)
    o       = a . down_proj_weight[e]           (down_proj_weight is [E, I, H])
y[t] = sum_k topk_weights[t, k] * o_{t,k}

The backward is the chain rule of that function (RFC section 2.2: dx,
d_up_proj_weight, d_down_proj_weight, d_topk_weights; topk_ids gets none):
    G      = dY[t] . down_proj_weight[e]^T       (the act_grad product)
    d_topk_weights[t, k] = <G, a>  (= <dY[t], o_{t,k}>)
    dA     = topk_weights[t, k] * G
    dg     = dA * u * s * (1 + g * (1 - s)),  s = sigmoid(g)   (SwiGLUGrad)
    du     = dA * silu(g)
    dH     = [dg | du]
    dx[t] += dH . up_proj_weight[e]^T                          (input_grad)
    d_up_proj_weight[e]   += x[t]^T dH                         (W1Grad)
    d_down_proj_weight[e] += (topk_weights[t, k] * a)^T dY[t]  (W2Grad)

Grouping slots by expert, permuting them and fusing stages changes only the
order of evaluation, so the oracle evaluates the definition directly: a loop
over tokens and their K slots for everything indexed by token, and, for the
weight gradients, the sum over the slots routed to each expert taken in
ascending slot order.

Modes
-----
``pure``      no intermediate rounding; float64 throughout.
``faithful``  the same arithmetic with bfloat16 round-to-nearest-even applied
              where a bfloat16 pipeline stores a value (the pages train in
              BF16 but do not list rounding points; these are the reading):
  R1 h   = bf16(x . W1[e])        (FP8 variant: bf16((xq . wq) * dsx * dsw))
  R2 a   = bf16(silu(g) * u)      from the rounded h
  R3 o   = bf16(a . W2[e])
  R4 y   = bf16(sum_k w * o)      (unless the output is float32)
  R5 dH  = bf16([dg | du])        from the rounded h and the unrounded G
  R6 dXp = bf16(dH . W1[e]^T)
  R7 dx  = bf16(sum_k dXp)
  R8 aw  = bf16(w * a)            the W2Grad operand
  R9 dW1 = bf16(sum x^T dH), dW2 = bf16(sum aw^T dY)
  d_topk_weights = sum_i G_i * a_i, float32 output, no rounding.

Admissible deviation (faithful mode)
------------------------------------
A pipeline that evaluates the value in front of a rounding point in float32
(any summation order) can land on the other side of a bfloat16 rounding
boundary when the exact value lies within its evaluation error of that
boundary; both neighbours are then correct results, and the choice propagates
downstream.  Next to every faithful value the oracle therefore carries
``dev``, a bound on how far an admissible result may lie from it:

  * at a value v with upstream deviation d_up, the float32 evaluation error is
    estimated as  eps = C_ACC * u * sqrt(n/2) * sqrt(sum_i t_i^2) + C_EL * u * |v|
    for a sum of n terms t_i (u = 2^-24; sqrt(n/2) sqrt(sum t^2) is the typical
    size of the partial sums' rounding errors; C_ACC = 8 is a wide margin) and
    d = d_up + eps;
  * rounding maps [v - d, v + d] onto the bfloat16 values between
    RNE(v - d) and RNE(v + d), so the rounded value's bound is
    max(|RNE(v + d) - RNE(v)|, |RNE(v) - RNE(v - d)|);
  * downstream, bounds propagate to first order, times C_PROP = 1.25 to cover
    the curvature over the few-ulp steps involved.  Through an elementwise
    formula the bound is sum_j |df/dv_j| d_j.  Through a reduction
    sum_i c_i delta_i over many upstream values, each delta_i is an open
    rounding decision of its own: it is 0 or +-d_i, decided by the evaluation
    noise of its own element, with a sign unrelated to c_i.  The bound there is
    min(sum_i |c_i| d_i, C_RMS sqrt(sum_i c_i^2 d_i^2)): the first term is the
    worst case (every decision open and all aligned), the second C_RMS = 3
    standard deviations of a sum of independent +-c_i d_i (every open decision
    taken, at random sign); the actual spread is smaller, since an open decision
    is taken only when the evaluation noise crosses the boundary.

dev is nonzero only on elements whose value (or an upstream value) lies within
its evaluation error of a bfloat16 rounding boundary; its size is pinned from
above against the tolerance (tests/test_oracle_dev.py).  Parity checks accept
|gpu - ref| <= atol + rtol |ref| + dev.  In pure mode dev is 0 and is not
computed.

The FP8 variant (``gmm1="fp8"``) quantises each token row and each
(expert, column) of the up-projection weight to E4M3 (see ``quant``) before
the up-projection; everything after R1, and the whole backward, stays as in
the bfloat16 mode.  The oracle sums the E4M3 products exactly.  The pages do
not say how precisely an FP8 product is accumulated; the reading is "as the
FP8 matrix instruction does it", and such instructions do not keep float32
accuracy: they sum small groups of products aligned to the group's largest
one with about 13 bits below it, then combine the group sums.  The
evaluation error of R1 in this variant is therefore taken as
C_F8 * 2^-24 * sqrt(sum of squared products) (in the accumulator's units),
with C_F8 = 2^12.  Errors of such an instruction measured on random E4M3 data
stay below 3300 * 2^-24 * sqrt(sum of squares), and below 1400 for Gaussian
data; a software model of it (groups of 8 products truncated 13 bits below the
group's largest, tests/test_oracle_dev.py) has median 230, 99th percentile 900
and maximum 2000 in the same units.  2^12 covers the worst of these with a
margin of 1.24.

The per-group variant (``gmm1="group"``) quantises tokens in groups of 128
along the hidden dimension and the weight in blocks of 128 rows per column
(see ``quant``).  Reading of the product: each group's E4M3 products are summed
as the FP8 instruction does (the bound above, per group), the group sum is
scaled by its token and weight descales in float32, and the scaled group sums
are added in float32 in group order; the oracle sums exactly and carries those
three errors in its deviation.

The FP8 backward (``bwd="fp8"``) runs the two products of the dX chain on E4M3,
with case 3's per-row dynamic rule applied to every operand: act_grad
G = (dYq . W2q^T) dsy dsw2 with dY quantised per token over H and W2[e] per
row i over H; input_grad dXp = (dHq . W1q^T) dsh dsw1 with dH quantised per
row over 2I and W1[e] per row h over 2I.  The weight gradients stay bfloat16.
dY and the weights are exact inputs, so their codes are exact.  dH is an
intermediate: where its bf16 decisions are open, its codes and its row descale
may come out otherwise (quant.quantize_rows_dev), and dXp's deviation carries
that.  The shared expert's backward stays bfloat16.

The MX variant (``gmm1="mx"``) quantises tokens and weights in blocks of 32
along the hidden dimension with a power-of-two scale per block (see
``quant``); the up-projection sums the dequantised products exactly, and the
same instruction-accumulation bound applies to them (the block scales are
powers of two, so they add no rounding of their own).
"""

import numpy as np

from .numerics import round_bf16, sigmoid, silu
from .quant import (GROUP, quantize_columns, quantize_columns_groups, quantize_columns_mx, quantize_rows,
                    quantize_rows_dev, quantize_rows_groups, quantize_rows_mx)
from .routing import check_ids

U32 = 2.0 ** -24     # unit roundoff of float32
C_ACC = 8.0          # margin on the typical accumulated rounding error of a float32 sum
C_EL = 8.0           # float32 evaluation error of an elementwise formula, in ulps
C_PROP = 1.25        # margin on first-order propagation (covers curvature over a few ulps)
C_F8 = 2.0 ** 12     # evaluation error of an FP8 matrix-instruction sum, in 2^-24 * sqrt(sum t^2)
C_RMS = 3.0          # standard deviations allowed for a sum of independent open rounding decisions


def acc_eps(sq_sum, n):
    """Evaluation-error estimate of a float32 sum of n terms whose squares sum to sq_sum."""
    return C_ACC * U32 * np.sqrt(max(n, 1) / 2.0) * np.sqrt(sq_sum)


def prop_sum(abs_sum, sq_sum):
    """Deviation of sum_i c_i delta_i, |delta_i| <= d_i, from abs_sum = sum |c_i| d_i and
    sq_sum = sum c_i^2 d_i^2: the smaller of the worst case and C_RMS standard deviations."""
    return np.minimum(abs_sum, C_RMS * np.sqrt(sq_sum))


def prop_matmul(d, c):
    """prop_sum over the contraction of d @ c (d: deviations, c: the coefficients)."""
    return prop_sum(d @ np.abs(c), (d * d) @ (c * c))


class MoEFFN:
    """One problem instance.  Inputs are float arrays holding exact bf16 values.

    x [T,H], topk_ids [T,K] int, topk_weights [T,K] float32,
    up_proj_weight [E,H,2I], down_proj_weight [E,I,H], dY [T,H] (optional).
    Weights are converted to float64 one expert at a time, on first use.
    Methods return values; the ``*_dev`` variants also return the admissible
    deviation bound described in the module text (zeros in pure mode).
    ``acc="f32"`` (pure mode only) evaluates every product and sum in float32.
    """

    def __init__(self, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
                 dY=None, mode="faithful", gmm1="bf16", shared_up_proj_weight=None, shared_down_proj_weight=None,
                 acc="f64", bwd="bf16"):
        if mode not in ("pure", "faithful"):
            raise ValueError(mode)
        if acc not in ("f64", "f32") or (acc == "f32" and mode != "pure"):
            raise ValueError("acc must be 'f64', or 'f32' in pure mode")
        # float type of every product and sum: float64 for parity; float32 only for
        # the pure mode's plain float32 per-token loop (a CPU timing baseline)
        self.ft = np.float64 if acc == "f64" else np.float32
        if gmm1 not in ("bf16", "fp8", "mx", "group"):
            raise ValueError(gmm1)
        if bwd not in ("bf16", "fp8"):
            raise ValueError(bwd)
        self.bwd = bwd
        self.x = np.asarray(x)
        self.ids = np.asarray(topk_ids, dtype=np.int64)
        self.w = np.asarray(topk_weights, dtype=np.float32).astype(self.ft)
        self.W1 = np.asarray(up_proj_weight)
        self.W2 = np.asarray(down_proj_weight)
        self.dY = None if dY is None else np.asarray(dY)
        self.mode, self.gmm1 = mode, gmm1
        self.faithful = mode == "faithful"
        self.T, self.H = self.x.shape
        self.K = self.ids.shape[1]
        self.E, _, two_i = self.W1.shape
        self.I = two_i // 2
        if self.ids.shape[0] != self.T or self.w.shape != self.ids.shape:
            raise ValueError("topk_ids / topk_weights must both be [T, K]")
        if two_i != 2 * self.I or self.W2.shape != (self.E, self.I, self.H):
            raise ValueError("weights must be [E,H,2I] and [E,I,H]")
        check_ids(self.ids, self.E)
        self._w1, self._w2, self._w1q, self._w2r, self._w1r = {}, {}, {}, {}, {}
        # Shared expert (RFC 6.1: an optional shared expert whose GMM1, SwiGLU and GMM2
        # run with the routed experts and whose output joins at the Combine).  Reading:
        # every token goes through it with weight 1; its output is added after the K
        # routed terms of the combine sum (and its dX after the K routed dXp terms).
        # It is evaluated as a one-expert, K = 1 problem of its own (bf16 products).
        self.shared = None
        if shared_up_proj_weight is not None:
            ws1 = np.asarray(shared_up_proj_weight)
            ws2 = np.asarray(shared_down_proj_weight)
            if ws1.ndim != 2 or ws1.shape[0] != self.H or ws2.shape != (ws1.shape[1] // 2, self.H):
                raise ValueError("shared weights must be [H, 2Is] and [Is, H]")
            self.shared = MoEFFN(self.x, np.zeros((self.T, 1), np.int64), np.ones((self.T, 1), np.float32),
                                 ws1[None], ws2[None], dY=self.dY, mode=mode, acc=acc)

    # -- helpers ---------------------------------------------------------------
    def _round(self, v, d):
        """Rounding point: (bf16(v), admissible deviation) in faithful mode; (v, None) in pure mode."""
        if not self.faithful:
            return v, None
        v = np.asarray(v, np.float64)
        r = round_bf16(v)
        dev = np.maximum(np.abs(round_bf16(v + d) - r), np.abs(r - round_bf16(v - d)))
        return r, dev

    def _W1(self, e):
        if e not in self._w1:
            self._w1[e] = self.W1[e].astype(self.ft)
        return self._w1[e]

    def _W2(self, e):
        if e not in self._w2:
            self._w2[e] = self.W2[e].astype(self.ft)
        return self._w2[e]

    def _sig(self, g):
        return sigmoid(g).astype(self.ft, copy=False)

    def _zeros_like(self, d, v):
        """d, or zeros shaped like v where d is None (pure mode)."""
        return np.zeros(np.shape(v)) if d is None else d

    def _W1q(self, e):
        if e not in self._w1q:
            if self.gmm1 == "mx":   # (q, e): dequantised value q * 2^e, blocks of 32 rows
                self._w1q[e] = quantize_columns_mx(self.W1[e])
            elif self.gmm1 == "group":  # (q, scale, descale [H / 128, 2I])
                self._w1q[e] = quantize_columns_groups(self.W1[e])
            else:                   # (q, scale, descale)
                self._w1q[e] = quantize_columns(self.W1[e])
        return self._w1q[e]

    def _W2r(self, e):
        """FP8 backward: W2[e] [I, H] quantised per row i (over H): (q, scale, descale)."""
        if e not in self._w2r:
            self._w2r[e] = quantize_rows(self.W2[e])
        return self._w2r[e]

    def _W1r(self, e):
        """FP8 backward: W1[e] [H, 2I] quantised per row h (over 2I): (q, scale, descale)."""
        if e not in self._w1r:
            self._w1r[e] = quantize_rows(self.W1[e])
        return self._w1r[e]

    def slots_of_expert(self, e):
        """Slots s = t*K + k routed to expert e, ascending."""
        return np.flatnonzero(self.ids.reshape(-1) == e)

    # -- per-slot stages (rows: any number of slots of ONE expert) ------------
    def up_dev(self, e, xrows, cols=None):
        """R1: h = x . W1[e] for the given rows (optionally a subset of columns)."""
        cols = slice(None) if cols is None else cols
        xr = np.asarray(xrows, self.ft)
        if self.gmm1 == "fp8":
            q, _, dsx = quantize_rows(xrows)
            wq, _, dsw = self._W1q(e)
            wqc = wq[:, cols]
            scale = dsx.astype(np.float64)[:, None] * dsw.astype(np.float64)[cols][None, :]
            h = (q @ wqc) * scale
            sq = (q * q) @ (wqc * wqc)
            eps = (acc_eps(sq, self.H) + C_F8 * U32 * np.sqrt(sq)) * scale + 2 * C_EL * U32 * np.abs(h)
        elif self.gmm1 == "group":
            q, _, dsx = quantize_rows_groups(xrows)
            wq, _, dsw = self._W1q(e)
            wqc, dswc = wq[:, cols], dsw[:, cols].astype(np.float64)
            ng = self.H // GROUP
            h = np.zeros((q.shape[0], wqc.shape[1]))
            eps_sq = np.zeros_like(h)
            terms_sq = np.zeros_like(h)
            for g in range(ng):                                     # groups in contraction order
                k = slice(g * GROUP, (g + 1) * GROUP)
                part = q[:, k] @ wqc[k]                             # exact sum of the group's E4M3 products
                sq = (q[:, k] * q[:, k]) @ (wqc[k] * wqc[k])
                sc = dsx[:, g].astype(np.float64)[:, None] * dswc[g][None, :]
                term = part * sc
                h += term
                terms_sq += term * term
                # the group sum's instruction error, then its scaling (two float32 products)
                eg = (acc_eps(sq, GROUP) + C_F8 * U32 * np.sqrt(sq)) * np.abs(sc) + 2 * C_EL * U32 * np.abs(term)
                eps_sq += eg * eg
            # The groups' errors are independent.  C_F8 bounds the error of a whole
            # instruction sum of any length in units of its sqrt(sum t^2), so the scaled
            # group errors combine in quadrature, without a further margin; then the
            # float32 running sum over the groups.
            eps = np.sqrt(eps_sq) + acc_eps(terms_sq, ng)
        elif self.gmm1 == "mx":
            q, ex = quantize_rows_mx(xrows)
            wq, ew = self._W1q(e)
            xd = q * np.repeat(np.exp2(ex), 32, axis=-1)           # dequantised tokens, exact
            wd = (wq * np.repeat(np.exp2(ew), 32, axis=0))[:, cols]  # dequantised weight columns, exact
            h = xd @ wd
            sq = (xd * xd) @ (wd * wd)
            eps = acc_eps(sq, self.H) + C_F8 * U32 * np.sqrt(sq)
        else:
            W = self._W1(e)[:, cols]
            h = xr @ W
            eps = acc_eps((xr * xr) @ (W * W), self.H) if self.faithful else None
        return self._round(h, eps)

    def up(self, e, xrows, cols=None):
        return self.up_dev(e, xrows, cols)[0]

    def hidden_dev(self, e, xrows, icols=None):
        """(g, u, a) and their deviations for gate columns ``icols`` (default all)."""
        if icols is None:
            h, hd = self.up_dev(e, xrows)
            n = self.I
        else:
            icols = np.asarray(icols)
            h, hd = self.up_dev(e, xrows, np.concatenate([icols, icols + self.I]))
            n = icols.size
        g, u = h[:, :n], h[:, n:]
        s = self._sig(g)
        v = g * s * u                                           # R2
        if not self.faithful:
            return (g, u, v), (None, None, None)
        gd, ud = hd[:, :n], hd[:, n:]
        d = C_PROP * (np.abs(u * (s + g * s * (1 - s))) * gd + np.abs(g * s) * ud) + C_EL * U32 * np.abs(v)
        a, ad = self._round(v, d)
        return (g, u, a), (gd, ud, ad)

    def hidden(self, e, xrows, icols=None):
        return self.hidden_dev(e, xrows, icols)[0]

    def down_dev(self, e, a, ad):
        """R3: o = a . W2[e]."""
        W2 = self._W2(e)
        v = a @ W2
        if not self.faithful:
            return v, None
        d = C_PROP * prop_matmul(ad, W2) + acc_eps((a * a) @ (W2 * W2), self.I)
        return self._round(v, d)

    def act_grad(self, e, dyrows, icols=None):
        """G = dY . W2[e]^T (unrounded) and its float32 evaluation error, for gate columns ``icols``.

        FP8 backward: dY rows quantised per token over H and W2[e] per row i over H
        (both exact inputs, so the codes are exact), G = (dYq . W2q^T) dsy dsw; the
        evaluation error carries the FP8 instruction's term."""
        if self.bwd == "fp8":
            q, _, dsy = quantize_rows(dyrows)
            wq, _, dsw = self._W2r(e)
            if icols is not None:
                wq, dsw = wq[np.asarray(icols)], dsw[np.asarray(icols)]
            sc = dsy.astype(np.float64)[:, None] * dsw.astype(np.float64)[None, :]
            G = (q @ wq.T) * sc
            if not self.faithful:
                return G, None
            sq = (q * q) @ (wq * wq).T
            return G, (acc_eps(sq, self.H) + C_F8 * U32 * np.sqrt(sq)) * sc + 2 * C_EL * U32 * np.abs(G)
        W2 = self._W2(e)
        W2 = W2 if icols is None else W2[np.asarray(icols)]
        dyr = np.asarray(dyrows, self.ft)
        if not self.faithful:
            return dyr @ W2.T, None
        return dyr @ W2.T, acc_eps((dyr * dyr) @ (W2 * W2).T, self.H)

    def input_grad_dev(self, e, dH, dHd):
        """R6: dXp = dH . W1[e]^T for the rows of dH (with deviations dHd).

        FP8 backward: dH rows quantised per row over 2I and W1[e] per row h over 2I,
        dXp = (dHq . W1q^T) dsh dsw.  dH is an intermediate: where its bf16 decisions
        are open, its E4M3 codes and its row descale may be others (quantize_rows_dev);
        code changes propagate like open decisions, a descale change scales the row."""
        if self.bwd != "fp8":
            W1 = self._W1(e)
            v = dH @ W1.T
            if not self.faithful:
                return v, None
            return self._round(v, C_PROP * prop_matmul(dHd, W1.T) + acc_eps((dH * dH) @ (W1 * W1).T, 2 * self.I))
        q, _, dsh = quantize_rows(dH)
        wq, _, dsw = self._W1r(e)
        sc = dsh.astype(np.float64)[:, None] * dsw.astype(np.float64)[None, :]
        v = (q @ wq.T) * sc
        if not self.faithful:
            return v, None
        dq, rel = quantize_rows_dev(dH, dHd)
        sq = (q * q) @ (wq * wq).T
        d = (C_PROP * (prop_matmul(dq, wq.T) * sc + rel[:, None] * np.abs(v))
             + (acc_eps(sq, 2 * self.I) + C_F8 * U32 * np.sqrt(sq)) * sc + 2 * C_EL * U32 * np.abs(v))
        return self._round(v, d)

    def swiglu_grad_dev(self, w, G, Ge, g, u, gd, ud):
        """SwiGLUGrad with dA = w G; R5: dH = [dg | du] and deviations."""
        s = self._sig(g)
        q = s * (1.0 + g * (1.0 - s))              # d silu / dg
        dA = w * G
        vg = dA * u * q
        vu = dA * g * s
        if not self.faithful:
            return (vg, None), (vu, None)
        dq = s * (1 - s) * (2.0 + g * (1.0 - 2.0 * s))  # d q / dg
        dvg = C_PROP * (np.abs(dA * u * dq) * gd + np.abs(dA * q) * ud + np.abs(w * u * q) * Ge) + C_EL * U32 * np.abs(vg)
        dvu = C_PROP * (np.abs(dA * q) * gd + np.abs(w * g * s) * Ge) + C_EL * U32 * np.abs(vu)
        return self._round(vg, dvg), self._round(vu, dvu)

    # -- forward ---------------------------------------------------------------
    def forward_dev(self, tokens=None, out_dtype="bf16"):
        """(y, dev) for the given tokens (default all), per-token loop over K slots."""
        toks = np.arange(self.T) if tokens is None else np.asarray(tokens)
        y = np.zeros((toks.size, self.H))
        yd = np.zeros((toks.size, self.H))
        if self.shared is not None:  # shared output o_s (R3 of the shared problem; its R4 of one term is exact)
            ys, ysd = self.shared.forward_dev(toks, out_dtype)
        for j, t in enumerate(toks):
            acc = np.zeros(self.H, self.ft)
            accd = np.zeros(self.H)
            accd2 = np.zeros(self.H)
            sq = np.zeros(self.H)
            for k in range(self.K):
                e = self.ids[t, k]
                (_, _, a), (_, _, ad) = self.hidden_dev(e, self.x[t:t + 1])
                o, od = self.down_dev(e, a, ad)
                acc = acc + self.w[t, k] * o[0]
                if self.faithful:
                    accd = accd + abs(self.w[t, k]) * od[0]
                    accd2 = accd2 + (self.w[t, k] * od[0]) ** 2
                    sq = sq + (self.w[t, k] * o[0]) ** 2
            nterm = self.K
            if self.shared is not None:
                acc, nterm = acc + ys[j], self.K + 1
                accd, accd2, sq = accd + ysd[j], accd2 + ysd[j] ** 2, sq + ys[j] ** 2
            if not self.faithful:
                y[j] = acc
            elif out_dtype == "bf16":
                y[j], yd[j] = self._round(acc, C_PROP * prop_sum(accd, accd2) + acc_eps(sq, nterm))      # R4
            else:
                y[j], yd[j] = acc, C_PROP * prop_sum(accd, accd2)
        return y, yd

    def forward(self, tokens=None, out_dtype="bf16"):
        return self.forward_dev(tokens, out_dtype)[0]

    def slot_intermediates(self, slots):
        """h (= [g|u]), a and o of the given slots, one row per slot (for checks)."""
        return self.slot_intermediates_dev(slots)[0]

    def slot_intermediates_dev(self, slots):
        slots = np.asarray(slots)
        out = [np.zeros((slots.size, 2 * self.I)), np.zeros((slots.size, self.I)), np.zeros((slots.size, self.H))]
        dev = [np.zeros_like(z) for z in out]
        for j, s in enumerate(slots):
            t, k = divmod(int(s), self.K)
            e = self.ids[t, k]
            (g, u, a), (gd, ud, ad) = self.hidden_dev(e, self.x[t:t + 1])
            o, od = self.down_dev(e, a, ad)
            out[0][j, :self.I], out[0][j, self.I:], out[1][j], out[2][j] = g[0], u[0], a[0], o[0]
            if self.faithful:
                dev[0][j, :self.I], dev[0][j, self.I:], dev[1][j], dev[2][j] = gd[0], ud[0], ad[0], od[0]
        return out, dev

    # -- backward --------------------------------------------------------------
    def backward_tokens_dev(self, tokens=None, out_dtype="bf16"):
        """((dx, d_topk_weights), (dx_dev, dw_dev)) for the given tokens."""
        if self.dY is None:
            raise ValueError("dY required")
        toks = np.arange(self.T) if tokens is None else np.asarray(tokens)
        dx = np.zeros((toks.size, self.H))
        dxd = np.zeros((toks.size, self.H))
        dw = np.zeros((toks.size, self.K))
        dwd = np.zeros((toks.size, self.K))
        if self.shared is not None:  # the shared dX rows (R6 of the shared problem)
            (dxs, _), (dxsd, _) = self.shared.backward_tokens_dev(toks, out_dtype)
        for j, t in enumerate(toks):
            acc = np.zeros(self.H, self.ft)
            accd = np.zeros(self.H)
            accd2 = np.zeros(self.H)
            sq = np.zeros(self.H)
            for k in range(self.K):
                e = self.ids[t, k]
                (g, u, a), (gd, ud, ad) = self.hidden_dev(e, self.x[t:t + 1])
                G, Ge = self.act_grad(e, self.dY[t:t + 1])
                dw[j, k] = float(np.sum(G * a))
                (dg, dgd), (du, dud) = self.swiglu_grad_dev(self.w[t, k], G, Ge, g, u, gd, ud)
                dH = np.concatenate([dg, du], axis=1)
                if not self.faithful:
                    acc = acc + self.input_grad_dev(e, dH, None)[0][0]
                    continue
                # d_topk_weights = sum_i G_i a_i: open decisions of a (ad) and the evaluation errors of G (Ge)
                dwd[j, k] = float(C_PROP * prop_sum(np.sum(np.abs(G) * ad + np.abs(a) * Ge),
                                                    np.sum((G * ad) ** 2 + (a * Ge) ** 2))
                                  + acc_eps(np.sum((G * a) ** 2), self.I))
                dHd = np.concatenate([dgd, dud], axis=1)
                xp, xpd = self.input_grad_dev(e, dH, dHd)                                          # R6
                acc = acc + xp[0]
                accd = accd + xpd[0]
                accd2 = accd2 + xpd[0] ** 2
                sq = sq + xp[0] ** 2
            nterm = self.K
            if self.shared is not None:
                acc, nterm = acc + dxs[j], self.K + 1
                accd, accd2, sq = accd + dxsd[j], accd2 + dxsd[j] ** 2, sq + dxs[j] ** 2
            if not self.faithful:
                dx[j] = acc
            elif out_dtype == "bf16":
                dx[j], dxd[j] = self._round(acc, C_PROP * prop_sum(accd, accd2) + acc_eps(sq, nterm))     # R7
            else:
                dx[j], dxd[j] = acc, C_PROP * prop_sum(accd, accd2)
        return (dx, dw), (dxd, dwd)

    def backward_tokens(self, tokens=None, out_dtype="bf16"):
        """(dx, d_topk_weights) for the given tokens, per-token loop over K slots."""
        return self.backward_tokens_dev(tokens, out_dtype)[0]

    def weight_grads_expert_dev(self, e, icols=None, out_dtype="bf16"):
        """Weight gradients of expert e restricted to gate columns ``icols``, with deviations.

        Returns ((dW1_gate[H, n], dW1_up[H, n], dW2_rows[n, H]), (their devs))
        where n = len(icols): columns i and I+i of d_up_proj_weight[e] and rows i
        of d_down_proj_weight[e].  The sum runs over the slots routed to e in
        ascending slot order; an expert with no slot gets exact zeros.
        """
        if self.dY is None:
            raise ValueError("dY required")
        icols = None if icols is None else np.asarray(icols)   # None: all columns, without an indexed copy
        slots = self.slots_of_expert(e)
        n = self.I if icols is None else icols.size
        if slots.size == 0:
            z = np.zeros((self.H, n))
            zr = np.zeros((n, self.H))
            return (z, z.copy(), zr), (z.copy(), z.copy(), zr.copy())
        t = slots // self.K
        k = slots % self.K
        xr = self.x[t].astype(self.ft)
        dyr = self.dY[t].astype(self.ft)
        w = self.w[t, k][:, None]
        (g, u, a), (gd, ud, ad) = self.hidden_dev(e, xr, icols)
        G, Ge = self.act_grad(e, dyr, icols)
        (dg, dgd), (du, dud) = self.swiglu_grad_dev(w, G, Ge, g, u, gd, ud)
        if not self.faithful:
            res = (xr.T @ dg, xr.T @ du, (w * a).T @ dyr)
            return res, tuple(np.broadcast_to(0.0, r.shape) for r in res)
        aw, awd = self._round(w * a, C_PROP * np.abs(w) * ad + C_EL * U32 * np.abs(w * a))    # R8
        m = slots.size
        res = [xr.T @ dg, xr.T @ du, aw.T @ dyr]                                      # R9
        devs = [C_PROP * prop_matmul(dgd.T, xr).T + acc_eps((xr * xr).T @ (dg * dg), m),
                C_PROP * prop_matmul(dud.T, xr).T + acc_eps((xr * xr).T @ (du * du), m),
                C_PROP * prop_matmul(awd.T, dyr) + acc_eps((aw * aw).T @ (dyr * dyr), m)]
        if out_dtype == "bf16":
            pairs = [self._round(v, d) for v, d in zip(res, devs)]
            res, devs = [p[0] for p in pairs], [p[1] for p in pairs]
        return tuple(res), tuple(devs)

    def weight_grads_expert(self, e, icols=None, out_dtype="bf16"):
        return self.weight_grads_expert_dev(e, icols, out_dtype)[0]

    def backward_dev(self, out_dtype="bf16"):
        """Full backward with deviations: ((dx, dw, dW1, dW2), (their devs))."""
        (dx, dw), (dxd, dwd) = self.backward_tokens_dev(None, out_dtype)
        dW1 = np.zeros((self.E, self.H, 2 * self.I), self.ft)
        dW2 = np.zeros((self.E, self.I, self.H), self.ft)
        if not self.faithful:   # no deviations: zero views, nothing allocated
            for e in range(self.E):
                (g, u, r), _ = self.weight_grads_expert_dev(e, None, out_dtype)
                dW1[e, :, :self.I], dW1[e, :, self.I:], dW2[e] = g, u, r
            return (dx, dw, dW1, dW2), (dxd, dwd, np.broadcast_to(0.0, dW1.shape), np.broadcast_to(0.0, dW2.shape))
        dW1d, dW2d = np.zeros_like(dW1), np.zeros_like(dW2)
        for e in range(self.E):
            (g, u, r), (gd, ud, rd) = self.weight_grads_expert_dev(e, None, out_dtype)
            dW1[e, :, :self.I], dW1[e, :, self.I:], dW2[e] = g, u, r
            dW1d[e, :, :self.I], dW1d[e, :, self.I:], dW2d[e] = gd, ud, rd
        return (dx, dw, dW1, dW2), (dxd, dwd, dW1d, dW2d)

    def backward(self, out_dtype="bf16"):
        """Full backward: dx [T,H], d_topk_weights [T,K], dW1 [E,H,2I], dW2 [E,I,H]."""
        return self.backward_dev(out_dtype)[0]

    # -- shared expert -----------------------------------------------------------
    def shared_weight_grads_dev(self, icols=None, out_dtype="bf16"):
        """Gradients of the shared weights, as weight_grads_expert_dev of its one-expert problem."""
        return self.shared.weight_grads_expert_dev(0, icols, out_dtype)

    def shared_backward_dev(self, out_dtype="bf16"):
        """((d_shared_up [H,2Is], d_shared_down [Is,H]), their devs)."""
        (g, u, r), (gd, ud, rd) = self.shared_weight_grads_dev(None, out_dtype)
        return (np.concatenate([g, u], 1), r), (np.concatenate([gd, ud], 1), rd)
