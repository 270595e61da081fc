"""Dynamic FP8 E4M3 quantisation of the oracle (test infrastructure).

Per-token dynamic quantisation follows "MoeDistributeDispatchV2", function
description, case 3 (quantMode 2): the row is taken to float32, its scale is
dstTypeMax / max|row|, the quantised row is the cast of row * scale, and the
scale that travels with the data is 1.0 / scale.  The page's formula writes
"CastToInt8" while its dtype lists give FP8 outputs; the reading here is a
cast to FP8 E4M3FN with dstTypeMax = 448.  The page does not say what happens
to an all-zero row (448 / 0); the reading is scale = 1 and a zero row.

The weight operand of an FP8 product must be FP8 too.  The pages quantise
only tokens; the reading for the up-projection weight is the same rule per
(expert, output column): scale = 448 / max over the hidden dimension.

Every step that decides a quantised code is done in float32, as the page's
"xFp32" states: float32 division for the scale, float32 product, then one
round-to-nearest-even into E4M3.
"""

import numpy as np

from .numerics import E4M3_MAX, round_e4m3


def _scale_from_absmax(absmax):
    absmax = np.asarray(absmax, dtype=np.float32)
    with np.errstate(divide="ignore"):
        scale = np.float32(E4M3_MAX) / absmax
    return np.where(absmax > 0, scale, np.float32(1.0)).astype(np.float32)


def quantize_rows(x):
    """Per-row dynamic quantisation of ``x`` [..., H].

    Returns (q, scale, descale): q holds the E4M3 values (as float64), scale is
    the float32 per-row factor and descale = 1 / scale in float32.
    """
    x32 = np.asarray(x, dtype=np.float32)
    scale = _scale_from_absmax(np.max(np.abs(x32), axis=-1))
    prod = (x32 * scale[..., None]).astype(np.float32)
    q = round_e4m3(prod.astype(np.float64))
    descale = (np.float32(1.0) / scale).astype(np.float32)
    return q, scale, descale


def quantize_columns(w):
    """Per-column dynamic quantisation of a weight ``w`` [H, N] (max over H)."""
    w32 = np.asarray(w, dtype=np.float32)
    scale = _scale_from_absmax(np.max(np.abs(w32), axis=0))
    prod = (w32 * scale[None, :]).astype(np.float32)
    q = round_e4m3(prod.astype(np.float64))
    descale = (np.float32(1.0) / scale).astype(np.float32)
    return q, scale, descale
