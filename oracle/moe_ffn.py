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

The FP8 variant (``gmm1="fp8"``) quantises each token row and each
(expert, column) of the up-projection weight to E4M3 (see ``quant``) before
the up-projection; everything after R1, and the whole backward, stays as in
the bfloat16 mode.
"""

import numpy as np

from .numerics import round_bf16, sigmoid, silu
from .quant import quantize_columns, quantize_rows
from .routing import check_ids


class MoEFFN:
    """One problem instance.  Inputs are float arrays holding exact bf16 values.

    x [T,H], topk_ids [T,K] int, topk_weights [T,K] float32,
    up_proj_weight [E,H,2I], down_proj_weight [E,I,H], dY [T,H] (optional).
    Weights are converted to float64 one expert at a time, on first use.
    """

    def __init__(self, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
                 dY=None, mode="faithful", gmm1="bf16"):
        if mode not in ("pure", "faithful"):
            raise ValueError(mode)
        if gmm1 not in ("bf16", "fp8"):
            raise ValueError(gmm1)
        self.x = np.asarray(x)
        self.ids = np.asarray(topk_ids, dtype=np.int64)
        self.w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
        self.W1 = np.asarray(up_proj_weight)
        self.W2 = np.asarray(down_proj_weight)
        self.dY = None if dY is None else np.asarray(dY)
        self.mode, self.gmm1 = mode, gmm1
        self.T, self.H = self.x.shape
        self.K = self.ids.shape[1]
        self.E, _, two_i = self.W1.shape
        self.I = two_i // 2
        if self.ids.shape[0] != self.T or self.w.shape != self.ids.shape:
            raise ValueError("topk_ids / topk_weights must both be [T, K]")
        if two_i != 2 * self.I or self.W2.shape != (self.E, self.I, self.H):
            raise ValueError("weights must be [E,H,2I] and [E,I,H]")
        check_ids(self.ids, self.E)
        self._w1, self._w2, self._w1q = {}, {}, {}

    # -- helpers ---------------------------------------------------------------
    def _r(self, v):
        return round_bf16(v) if self.mode == "faithful" else np.asarray(v, np.float64)

    def _W1(self, e):
        if e not in self._w1:
            self._w1[e] = self.W1[e].astype(np.float64)
        return self._w1[e]

    def _W2(self, e):
        if e not in self._w2:
            self._w2[e] = self.W2[e].astype(np.float64)
        return self._w2[e]

    def _W1q(self, e):
        if e not in self._w1q:
            self._w1q[e] = quantize_columns(self.W1[e])  # (q, scale, descale)
        return self._w1q[e]

    def slots_of_expert(self, e):
        """Slots s = t*K + k routed to expert e, ascending."""
        return np.flatnonzero(self.ids.reshape(-1) == e)

    # -- per-slot stages (rows: any number of slots of ONE expert) ------------
    def up(self, e, xrows, cols=None):
        """R1: h = x . W1[e] for the given rows (optionally a subset of columns)."""
        cols = slice(None) if cols is None else cols
        if self.gmm1 == "fp8":
            q, _, dsx = quantize_rows(xrows)
            wq, _, dsw = self._W1q(e)
            acc = q @ wq[:, cols]
            h = acc * dsx.astype(np.float64)[:, None] * dsw.astype(np.float64)[cols][None, :]
        else:
            h = np.asarray(xrows, np.float64) @ self._W1(e)[:, cols]
        return self._r(h)

    def swiglu(self, g, u):
        """R2: a = silu(g) * u."""
        return self._r(silu(g) * u)

    def hidden(self, e, xrows, icols=None):
        """Return (g, u, a) of the rows for gate columns ``icols`` (default all)."""
        icols = np.arange(self.I) if icols is None else np.asarray(icols)
        h = self.up(e, xrows, np.concatenate([icols, icols + self.I]))
        n = icols.size
        g, u = h[:, :n], h[:, n:]
        return g, u, self.swiglu(g, u)

    def down(self, e, a):
        """R3: o = a . W2[e]."""
        return self._r(a @ self._W2(e))

    def act_grad(self, e, dyrows, icols=None):
        """G = dY . W2[e]^T (unrounded) for gate columns ``icols``."""
        W2 = self._W2(e)
        W2 = W2 if icols is None else W2[np.asarray(icols)]
        return np.asarray(dyrows, np.float64) @ W2.T

    def swiglu_grad(self, dA, g, u):
        """SwiGLUGrad, R5: dH = [dg | du]."""
        s = sigmoid(g)
        dg = dA * u * s * (1.0 + g * (1.0 - s))
        du = dA * g * s
        return self._r(dg), self._r(du)

    # -- forward ---------------------------------------------------------------
    def forward(self, tokens=None, out_dtype="bf16"):
        """y for the given tokens (default all), per-token loop over K slots."""
        toks = np.arange(self.T) if tokens is None else np.asarray(tokens)
        y = np.zeros((toks.size, self.H))
        for j, t in enumerate(toks):
            acc = np.zeros(self.H)
            for k in range(self.K):
                e = self.ids[t, k]
                _, _, a = self.hidden(e, self.x[t:t + 1])
                o = self.down(e, a)[0]
                acc = acc + self.w[t, k] * o
            y[j] = round_bf16(acc) if (out_dtype == "bf16" and self.mode == "faithful") else acc
        return y

    def slot_intermediates(self, slots):
        """h (= [g|u]), a and o of the given slots, one row per slot (for checks)."""
        slots = np.asarray(slots)
        h = np.zeros((slots.size, 2 * self.I))
        a = np.zeros((slots.size, self.I))
        o = np.zeros((slots.size, self.H))
        for j, s in enumerate(slots):
            t, k = divmod(int(s), self.K)
            e = self.ids[t, k]
            g, u, aa = self.hidden(e, self.x[t:t + 1])
            h[j, :self.I], h[j, self.I:], a[j] = g[0], u[0], aa[0]
            o[j] = self.down(e, aa)[0]
        return h, a, o

    # -- backward --------------------------------------------------------------
    def backward_tokens(self, tokens=None, out_dtype="bf16"):
        """(dx, d_topk_weights) for the given tokens, per-token loop over K slots."""
        if self.dY is None:
            raise ValueError("dY required")
        toks = np.arange(self.T) if tokens is None else np.asarray(tokens)
        dx = np.zeros((toks.size, self.H))
        dw = np.zeros((toks.size, self.K))
        for j, t in enumerate(toks):
            acc = np.zeros(self.H)
            for k in range(self.K):
                e = self.ids[t, k]
                g, u, a = self.hidden(e, self.x[t:t + 1])
                G = self.act_grad(e, self.dY[t:t + 1])
                dw[j, k] = float(np.sum(G * a))
                dg, du = self.swiglu_grad(self.w[t, k] * G, g, u)
                dH = np.concatenate([dg, du], axis=1)
                dxp = self._r(dH @ self._W1(e).T)[0]             # R6
                acc = acc + dxp
            dx[j] = round_bf16(acc) if (out_dtype == "bf16" and self.mode == "faithful") else acc
        return dx, dw

    def weight_grads_expert(self, e, icols=None, out_dtype="bf16"):
        """Weight gradients of expert e restricted to gate columns ``icols``.

        Returns (dW1_gate[H, n], dW1_up[H, n], dW2_rows[n, H]) where n =
        len(icols): columns i and I+i of d_up_proj_weight[e] and rows i of
        d_down_proj_weight[e].  The sum runs over the slots routed to e in
        ascending slot order; an expert with no slot gets exact zeros.
        """
        if self.dY is None:
            raise ValueError("dY required")
        icols = np.arange(self.I) if icols is None else np.asarray(icols)
        slots = self.slots_of_expert(e)
        n = icols.size
        if slots.size == 0:
            z = np.zeros((self.H, n))
            return z, z.copy(), np.zeros((n, self.H))
        t = slots // self.K
        k = slots % self.K
        xr = self.x[t].astype(np.float64)
        dyr = self.dY[t].astype(np.float64)
        w = self.w[t, k][:, None]
        g, u, a = self.hidden(e, xr, icols)
        G = self.act_grad(e, dyr, icols)
        dg, du = self.swiglu_grad(w * G, g, u)
        aw = self._r(w * a)                                       # R8
        dW1g = xr.T @ dg                                          # R9
        dW1u = xr.T @ du
        dW2r = aw.T @ dyr
        if out_dtype == "bf16" and self.mode == "faithful":
            dW1g, dW1u, dW2r = round_bf16(dW1g), round_bf16(dW1u), round_bf16(dW2r)
        return dW1g, dW1u, dW2r

    def backward(self, out_dtype="bf16"):
        """Full backward: dx [T,H], d_topk_weights [T,K], dW1 [E,H,2I], dW2 [E,I,H]."""
        dx, dw = self.backward_tokens(None, out_dtype)
        dW1 = np.zeros((self.E, self.H, 2 * self.I))
        dW2 = np.zeros((self.E, self.I, self.H))
        for e in range(self.E):
            g, u, r = self.weight_grads_expert(e, None, out_dtype)
            dW1[e, :, :self.I], dW1[e, :, self.I:], dW2[e] = g, u, r
        return dx, dw, dW1, dW2
