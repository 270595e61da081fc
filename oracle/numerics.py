"""Rounding primitives of the oracle (test infrastructure).

The pages fix bfloat16 as the training precision ("MoE multicore parallel
usage guide", Torch managed API: Torch BF16 training) and name FP8 E4M3FN as a
token dtype of the dispatch quantisation ("MoeDistributeDispatchV2", parameter
table, x / expandXOut).  Neither page states a rounding mode; the reading used
throughout is IEEE round-to-nearest-even.

Both roundings are written directly from the format definitions, working on
float64 values so that a float64 result is rounded once (never via float32):

* bfloat16: 8 exponent bits (bias 127), 7 stored fraction bits; normal
  numbers start at 2**-126, below that the spacing is fixed at 2**-133;
  largest finite value (2 - 2**-7) * 2**127; overflow gives infinity.
* FP8 E4M3FN (OCP): 4 exponent bits (bias 7), 3 fraction bits; normal numbers
  start at 2**-6, subnormal spacing 2**-9; largest finite value 448; there is
  no infinity, and this oracle saturates to +-448 (the dispatch formula's
  scale keeps every quantised value within +-448 anyway).
"""

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
E4M3_MAX = 448.0


def _round_to_grid(v, frac_bits, min_normal_exp):
    """Round float64 ``v`` to the nearest value with ``frac_bits`` fraction bits.

    The spacing of representable values next to ``v`` is
    2**(max(floor(log2|v|), min_normal_exp) - frac_bits); dividing by that
    power of two is exact, so ``np.rint`` (round half to even) performs the
    whole rounding in one step.
    """
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v)
    vf = v[fin]
    _, e = np.frexp(vf)                      # vf = m * 2**e with 0.5 <= |m| < 1
    lead = np.maximum(e - 1, min_normal_exp)  # exponent of the leading bit
    quantum = np.ldexp(np.ones_like(vf), lead - frac_bits)
    out[fin] = np.rint(vf / quantum) * quantum
    return out


def round_bf16(v):
    """Nearest bfloat16 value (ties to even) of float64 ``v``, as float64."""
    r = _round_to_grid(v, 7, -126)
    over = np.isfinite(r) & (np.abs(r) > BF16_MAX)
    r[over] = np.copysign(np.inf, r[over])
    return r


def round_e4m3(v):
    """Nearest FP8 E4M3FN value (ties to even, saturating at +-448) of ``v``."""
    r = _round_to_grid(v, 3, -6)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def bf16_bits_to_f64(bits):
    """Exact float64 value of bfloat16 bit patterns given as uint16."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def sigmoid(g):
    """Logistic function 1 / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def silu(g):
    """SiLU (swish): g * sigmoid(g)."""
    return np.asarray(g, dtype=np.float64) * sigmoid(g)
