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
    """448 / absmax in float32; 1 for an all-zero row.  The page's formula
    overflows float32 when 0 < absmax < ~1.3e-36 (bfloat16 holds values down to
    ~9e-41); the reading is that the quotient is clamped to the largest finite
    float32, which keeps the codes finite."""
    absmax = np.asarray(absmax, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        scale = np.minimum(np.float32(E4M3_MAX) / absmax, np.finfo(np.float32).max)
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


# ----------------------------------------------------------------------------- MX
# MoeDistributeDispatchV2, case 5 (quantMode 4, "mx"): the shared exponent of a
# block is floor(log2(max)) - emax, where emax is the exponent of the target
# type's largest normal value (E4M3: 448 = 1.75 * 2^8, emax = 8); the block's
# scale is 2^sharedExp and the codes are the FP8 cast of X / scale.
# Readings (the page leaves them open):
# * the block is 32 consecutive elements along the contraction dimension (the
#   OCP MX block size; the page gives none), and "max(x)" is max |x| of the block;
# * the cast saturates at +-448 (X / scale reaches up to 2^9 - ulp, above the
#   largest E4M3 value), rounding to nearest even below that;
# * the exponent is stored as E8M0 (its range is 2^-127 .. 2^127; exponents
#   outside are clamped); an all-zero block gets the smallest, 2^-127;
# * the factor that travels with the codes is the scale itself (X ~ code *
#   2^sharedExp); the page's "1.0/dynamicScales" is case 3's convention, where
#   the scale multiplies X.
# The up-projection weight gets the same rule per (expert, column, block of 32
# rows along the hidden dimension).

MX_BLOCK = 32
E4M3_EMAX = 8


def mx_exponent(absmax):
    """Shared block exponent floor(log2(absmax)) - 8, clamped to [-127, 127] (-127 for 0)."""
    a = np.asarray(absmax, dtype=np.float64)
    _, ex = np.frexp(a)                       # a = m * 2^ex with 0.5 <= m < 1: floor(log2 a) = ex - 1
    e = ex.astype(np.int64) - 1 - E4M3_EMAX
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_rows_mx(x):
    """MX quantisation of ``x`` [..., H] in blocks of 32 along H.

    Returns (q, e): q the E4M3 values [..., H] (float64), e the block exponents
    [..., H / 32] (int64); the dequantised value is q * 2^e.
    """
    x = np.asarray(x, dtype=np.float64)
    H = x.shape[-1]
    if H % MX_BLOCK:
        raise ValueError("H must be a multiple of %d" % MX_BLOCK)
    xb = x.reshape(x.shape[:-1] + (H // MX_BLOCK, MX_BLOCK))
    e = mx_exponent(np.max(np.abs(xb), axis=-1))
    q = round_e4m3(xb / np.exp2(e)[..., None].astype(np.float64))
    return q.reshape(x.shape), e


def quantize_columns_mx(w):
    """MX quantisation of a weight ``w`` [H, N] in blocks of 32 rows per column.

    Returns (q [H, N], e [H / 32, N])."""
    w = np.asarray(w, dtype=np.float64)
    H, N = w.shape
    if H % MX_BLOCK:
        raise ValueError("H must be a multiple of %d" % MX_BLOCK)
    wb = w.reshape(H // MX_BLOCK, MX_BLOCK, N)
    e = mx_exponent(np.max(np.abs(wb), axis=1))
    q = round_e4m3(wb / np.exp2(e)[:, None, :].astype(np.float64))
    return q.reshape(H, N), e


# ---------------------------------------------------------------- per group
# MoeDistributeDispatchV2, case 4 (quantMode 3, "pergroup" / "pertile" dynamic
# quantisation): the same formula as case 3 (scale = dstTypeMax / max|x|, codes
# = cast(x * scale), 1 / scale travelling with them), taken over a group of a
# token row instead of the whole row.  Readings (the page leaves them open):
# * a group is 128 consecutive elements along the hidden (contraction)
#   dimension; the page gives no size, and 128 divides every hidden size here;
# * the cast and the all-zero rule are case 3's (E4M3, 448; an all-zero group
#   gets scale 1 and zero codes);
# * the up-projection weight is quantised by the same rule per (expert, column,
#   block of 128 rows along the hidden dimension), so each group of the
#   contraction has one token scale and one weight scale per output column.

GROUP = 128


def quantize_rows_groups(x, group=GROUP):
    """Per-group dynamic quantisation of ``x`` [..., H] in groups of ``group`` along H.

    Returns (q [..., H] E4M3 values as float64, scale [..., H / group] float32,
    descale = 1 / scale float32)."""
    x32 = np.asarray(x, dtype=np.float32)
    H = x32.shape[-1]
    if H % group:
        raise ValueError("H must be a multiple of %d" % group)
    xg = x32.reshape(x32.shape[:-1] + (H // group, group))
    scale = _scale_from_absmax(np.max(np.abs(xg), axis=-1))
    prod = (xg * scale[..., None]).astype(np.float32)
    q = round_e4m3(prod.astype(np.float64)).reshape(x32.shape)
    descale = (np.float32(1.0) / scale).astype(np.float32)
    return q, scale, descale


def quantize_columns_groups(w, group=GROUP):
    """Per-(block of ``group`` rows, column) quantisation of a weight ``w`` [H, N].

    Returns (q [H, N], scale [H / group, N], descale [H / group, N])."""
    w32 = np.asarray(w, dtype=np.float32)
    H, N = w32.shape
    if H % group:
        raise ValueError("H must be a multiple of %d" % group)
    wg = w32.reshape(H // group, group, N)
    scale = _scale_from_absmax(np.max(np.abs(wg), axis=1))
    prod = (wg * scale[:, None, :]).astype(np.float32)
    q = round_e4m3(prod.astype(np.float64)).reshape(H, N)
    descale = (np.float32(1.0) / scale).astype(np.float32)
    return q, scale, descale


# ----------------------------------------------------------- admissible rows
def quantize_rows_dev(v, d):
    """Deviation bounds of the per-row E4M3 quantisation of rows ``v`` [n, L] whose
    elements may each lie anywhere in [v - d, v + d] (the open bf16 decisions of an
    intermediate, see moe_ffn): returns (dq, rel), with dq [n, L] the largest change
    of each E4M3 code and rel [n] the largest relative change of the row's float32
    descale 1 / scale, over every admissible row.

    The row maximum of an admissible row lies in [m_lo, m_hi] (m_lo = max(|v| - d),
    m_hi = max(|v| + d)), so its scale lies between the scales of those two (the
    largest finite float32 if m_lo is 0); each code is a monotone function of
    float32(v' * s'), so its extremes are at the corners of that box.
    """
    v = np.asarray(v, np.float64)
    d = np.asarray(d, np.float64)
    a = np.abs(v)
    m = a.max(axis=-1)
    m_lo = np.maximum(a - d, 0.0).max(axis=-1)
    m_hi = (a + d).max(axis=-1)
    fmax = np.float32(np.finfo(np.float32).max)
    s = _scale_from_absmax(m)
    s_lo = _scale_from_absmax(m_hi)
    s_hi = np.where(m_lo > 0, _scale_from_absmax(m_lo), fmax).astype(np.float32)
    s_hi = np.where(m_hi > 0, s_hi, s)                       # an all-zero row stays all-zero
    q = round_e4m3((v.astype(np.float32) * s[..., None]).astype(np.float64))
    corners = [(np.float32(x) * sc[..., None]).astype(np.float64)
               for x in ((v - d).astype(np.float32), (v + d).astype(np.float32)) for sc in (s_lo, s_hi)]
    lo = round_e4m3(np.minimum.reduce(corners))
    hi = round_e4m3(np.maximum.reduce(corners))
    dq = np.maximum(np.abs(hi - q), np.abs(q - lo))
    with np.errstate(divide="ignore", over="ignore"):
        ds = (np.float32(1.0) / s).astype(np.float64)
        ds_a = (np.float32(1.0) / s_lo).astype(np.float64)
        ds_b = (np.float32(1.0) / s_hi).astype(np.float64)
    rel = np.maximum(np.abs(ds_a - ds), np.abs(ds_b - ds)) / ds
    return dq, rel
