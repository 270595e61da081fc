"""Pins of the oracle's dynamic FP8 E4M3 quantisation and of the FP8 up-projection."""

import numpy as np
import torch

from oracle.moe_ffn import MoEFFN
from oracle.numerics import round_bf16, round_e4m3
from oracle.quant import quantize_columns, quantize_rows


def test_row_quant_matches_torch_float32_ops_and_cast():
    rng = np.random.default_rng(0)
    x = round_bf16(rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    q, scale, descale = quantize_rows(x)
    tx = torch.from_numpy(x)
    tscale = torch.tensor(448.0, dtype=torch.float32) / tx.abs().amax(dim=1)
    assert np.array_equal(scale, tscale.numpy())
    tq = (tx * tscale[:, None]).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(q, tq)
    assert np.array_equal(descale, (1.0 / tscale).numpy())
    # the largest magnitude of every row lands on +-448
    assert np.all(np.abs(q).max(axis=1) == 448.0)


def test_column_quant_matches_torch_float32_ops_and_cast():
    rng = np.random.default_rng(1)
    w = round_bf16(rng.standard_normal((128, 96)) / 11.3).astype(np.float32)
    q, scale, descale = quantize_columns(w)
    tw = torch.from_numpy(w)
    tscale = torch.tensor(448.0, dtype=torch.float32) / tw.abs().amax(dim=0)
    assert np.array_equal(scale, tscale.numpy())
    assert np.array_equal(q, (tw * tscale[None, :]).to(torch.float8_e4m3fn).to(torch.float64).numpy())
    assert np.array_equal(descale, (1.0 / tscale).numpy())


def test_zero_row_gets_unit_scale():
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = -2.0
    q, scale, descale = quantize_rows(x)
    assert scale[0] == 1.0 and scale[2] == 1.0 and descale[0] == 1.0
    assert np.all(q[0] == 0) and q[1, 5] == -448.0


def test_fp8_up_projection_equals_bf16_when_quantisation_is_exact():
    """Rows and columns whose entries are +-2^j with max 1 quantise exactly (scale 448).

    Then (xq . wq) * (1/448) * (1/448) equals x . W1 up to the float32 rounding of
    1/448, so the FP8 and bf16 up-projections agree to ~1e-7 in pure mode.  Each
    column has its own maximum, so a misapplied per-column scale would show.
    """
    rng = np.random.default_rng(2)
    T, H, I, E, K = 6, 32, 8, 2, 2
    x = np.where(rng.random((T, H)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (T, H))
    x[:, 0] = 1.0
    W1 = np.where(rng.random((E, H, 2 * I)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (E, H, 2 * I))
    colmax = 2.0 ** -rng.integers(0, 3, (E, 1, 2 * I))
    W1 = W1 * colmax
    W1[:, 0, :] = colmax[:, 0, :]
    W2 = rng.standard_normal((E, I, H))
    ids = np.array([[0, 1]] * T)
    w = np.full((T, K), 0.5, np.float32)
    y8 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="fp8").forward()
    y16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16").forward()
    assert np.allclose(y8, y16, rtol=1e-6, atol=1e-6)


def test_fp8_up_projection_error_is_bounded():
    """Generic data: each E4M3 code has relative error <= 2^-4, so h moves by a bounded amount."""
    rng = np.random.default_rng(3)
    T, H, I, E, K = 8, 64, 16, 3, 2
    x = round_bf16(rng.standard_normal((T, H)))
    W1 = round_bf16(rng.standard_normal((E, H, 2 * I)) / 8)
    W2 = round_bf16(rng.standard_normal((E, I, H)) / 4)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    w = np.full((T, K), 0.5, np.float32)
    m8 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="fp8")
    m16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")
    for e in range(E):
        h8 = m8.up(e, x)
        h16 = m16.up(e, x)
        bound = (2 * 2.0 ** -4 + 2.0 ** -8) * (np.abs(x) @ np.abs(W1[e]))
        assert np.all(np.abs(h8 - h16) <= bound)


# ----------------------------------------------------------------------------- MX (Dispatch case 5)
from oracle.quant import mx_exponent, quantize_columns_mx, quantize_rows_mx  # noqa: E402


def test_mx_closed_forms():
    """Block exponent floor(log2 max|x|) - 8 (E4M3's emax), codes X / 2^e, saturating at 448."""
    x = np.zeros((1, 8 * 32))
    x[0, 0:32] = 0.25                      # max 2^-2: e = -10, every code 256
    x[0, 32] = 1.5 * 2.0 ** 5              # max 1.5 * 2^5: e = -3, code 384 exactly
    x[0, 33] = -2.0 ** 5                   # same block: code -256
    x[0, 64] = 1.875 * 2.0 ** 3            # max 1.875 * 2^3: e = -5, 480 saturates to 448
    x[0, 96] = 1.75 * 2.0 ** -3            # 1.75 * 256 = 448: representable, no saturation
    # block 4 stays zero: e = -127, codes 0
    x[0, 160] = 2.0 ** -140                # e clamped to -127; 2^-13 rounds to code 0
    x[0, 192] = 2.0 ** 130                 # e = 122, code 256
    x[0, 193] = 2.0 ** 120                 # 2^120 / 2^122 = 0.25: an exact E4M3 value
    x[0, 224] = 3.0                        # max 3: e = -7, 3 / 2^-7 = 384
    x[0, 225] = 3.0 * 2.0 ** -12           # 384 * 2^-12 = 0.09375 = 0.75 * 2^-3: exact
    x[0, 226] = 3.0 * 2.0 ** -19           # 384 * 2^-19 = 0.000732...: below 2^-10 -> rounds to 0
    q, e = quantize_rows_mx(x)
    assert e.tolist() == [[-10, -3, -5, -11, -127, -127, 122, -7]]
    assert np.all(q[0, 0:32] == 256)
    assert q[0, 32] == 384 and q[0, 33] == -256 and np.all(q[0, 34:64] == 0)
    assert q[0, 64] == 448 and q[0, 96] == 448
    assert np.all(q[0, 128:192] == 0)
    assert q[0, 192] == 256 and q[0, 193] == 0.25
    assert q[0, 224] == 384 and q[0, 225] == 0.09375 and q[0, 226] == 0
    assert mx_exponent(0.0) == -127 and mx_exponent(2.0 ** 200) == 127 and mx_exponent(511.0) == 0


def test_mx_rows_match_torch_cast():
    """Codes equal torch's float8_e4m3fn cast of the block-scaled values clamped to +-448,
    with the exponent from torch.frexp; blocks span many magnitudes."""
    rng = np.random.default_rng(5)
    x = round_bf16(rng.standard_normal((16, 256)) * np.exp2(rng.integers(-30, 30, (16, 256 // 32))).repeat(32, 1))
    q, e = quantize_rows_mx(x)
    tx = torch.from_numpy(x).reshape(16, 8, 32)
    _, ex = torch.frexp(tx.abs().amax(dim=2))
    te = torch.clamp(ex.to(torch.int64) - 9, -127, 127)
    assert np.array_equal(e, te.numpy())
    scaled = tx / torch.exp2(te.to(torch.float64))[..., None]
    tq = torch.clamp(scaled, -448, 448).to(torch.float8_e4m3fn).to(torch.float64).reshape(16, 256)
    assert np.array_equal(q, tq.numpy())
    # dequantisation error: half an E4M3 step at the element's binade, or the
    # saturation at 448 * 2^e (block maxima up to 512 * 2^e), plus half the
    # smallest subnormal step of the block
    deq = q * np.exp2(e).repeat(32, 1)
    s = np.exp2(e).repeat(32, 1)
    bound = np.maximum(2.0 ** -4 * np.abs(x), np.abs(x) - 448 * s) + s * 2.0 ** -10
    assert np.all(np.abs(deq - x) <= bound)
    assert np.any(np.abs(x) > 448 * s)      # saturation occurs in this data


def test_mx_columns_are_row_blocks_per_column():
    rng = np.random.default_rng(6)
    w = round_bf16(rng.standard_normal((96, 10)) * np.exp2(rng.integers(-8, 8, (3, 1, 10))).repeat(32, 0).reshape(96, 10))
    q, e = quantize_columns_mx(w)
    qt, et = quantize_rows_mx(w.T)          # the same rule, transposed
    assert np.array_equal(q, qt.T) and np.array_equal(e, et.T)
    assert e.shape == (3, 10)


def test_mx_up_projection_exact_when_blocks_are_representable():
    """x = code * 2^e per block, with the block's largest |code| in [256, 448], quantises back
    exactly; likewise W1 per (32-row block, column).  Then the MX up-projection equals
    the bf16 one exactly (pure mode), so a misplaced block exponent would show."""
    rng = np.random.default_rng(7)
    T, H, I, E, K = 5, 64, 8, 2, 2
    codes = np.array([c for c in np.arange(0, 449, 0.125) if np.array_equal(
        np.asarray([c]), np.asarray([float(torch.tensor(c).to(torch.float8_e4m3fn).to(torch.float64))]))])

    def block_values(shape):
        return rng.choice(codes, shape) * np.where(rng.random(shape) < 0.5, -1.0, 1.0)

    x = block_values((T, H))
    x[:, 0], x[:, 32] = 320.0, -448.0               # block maxima in [256, 448]
    ex = rng.integers(-12, 6, (T, H // 32))
    x = x * np.exp2(ex).repeat(32, 1)
    W1 = block_values((E, H, 2 * I))
    W1[:, 0, :], W1[:, 32, :] = 256.0, 416.0
    ew = rng.integers(-14, 0, (E, H // 32, 2 * I))
    W1 = W1 * np.exp2(ew).repeat(32, 1)
    W2 = rng.standard_normal((E, I, H))
    ids = np.array([[0, 1]] * T)
    w = np.full((T, K), 0.5, np.float32)
    mx = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="mx")
    bf = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")
    for e in range(E):
        assert np.array_equal(mx.up(e, x), bf.up(e, x))
    q, e_ = quantize_rows_mx(x)
    assert np.array_equal(e_, ex) and np.array_equal(q * np.exp2(e_).repeat(32, 1), x)
    for e in range(E):
        qw, e_ = quantize_columns_mx(W1[e])
        assert np.array_equal(e_, ew[e]) and np.array_equal(qw * np.exp2(e_).repeat(32, 0), W1[e])


def test_mx_up_projection_error_is_bounded():
    """Generic data: every dequantised element is within max(2^-4 |v|, |v| - 448 2^e) + 2^(e-10) of v."""
    rng = np.random.default_rng(8)
    T, H, I, E, K = 8, 64, 16, 3, 2
    x = round_bf16(rng.standard_normal((T, H)) * np.exp2(rng.integers(-4, 4, (T, 2))).repeat(32, 1))
    W1 = round_bf16(rng.standard_normal((E, H, 2 * I)) / 8)
    W2 = round_bf16(rng.standard_normal((E, I, H)) / 4)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    w = np.full((T, K), 0.5, np.float32)
    mmx = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="mx")
    m16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")
    def dev(v, s):
        return np.maximum(2.0 ** -4 * np.abs(v), np.abs(v) - 448 * s) + s * 2.0 ** -10

    _, ex = quantize_rows_mx(x)
    dx = dev(x, np.exp2(ex).repeat(32, 1))
    for e in range(E):
        _, ew = quantize_columns_mx(W1[e])
        dw = dev(W1[e], np.exp2(ew).repeat(32, 0))
        bound = dx @ (np.abs(W1[e]) + dw) + np.abs(x) @ dw
        assert np.all(np.abs(mmx.up(e, x) - m16.up(e, x)) <= bound)


# ----------------------------------------------------------------------------- per group (Dispatch case 4)
from oracle.quant import GROUP, quantize_columns_groups, quantize_rows_groups  # noqa: E402


def test_group_quant_matches_torch_float32_ops_and_cast():
    """Every 128-element group of a row gets 448 / max|group| in float32 and the E4M3 cast of
    x * scale; the groups are independent (magnitudes differ by up to 2^12 across them)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 512)) * np.exp2(rng.integers(-6, 6, (16, 4))).repeat(GROUP, 1)
    x = round_bf16(x).astype(np.float32)
    q, scale, descale = quantize_rows_groups(x)
    tx = torch.from_numpy(x).reshape(16, 4, GROUP)
    tscale = torch.tensor(448.0, dtype=torch.float32) / tx.abs().amax(dim=2)
    assert np.array_equal(scale, tscale.numpy())
    tq = (tx * tscale[:, :, None]).to(torch.float8_e4m3fn).to(torch.float64).reshape(16, 512).numpy()
    assert np.array_equal(q, tq)
    assert np.array_equal(descale, (1.0 / tscale).numpy())
    # the largest magnitude of every group lands on +-448
    assert np.all(np.abs(q.reshape(16, 4, GROUP)).max(axis=2) == 448.0)


def test_group_quant_special_cases():
    """One group spanning the row is the per-token rule; an all-zero group gets scale 1."""
    rng = np.random.default_rng(12)
    x = round_bf16(rng.standard_normal((5, 256))).astype(np.float32)
    q1, s1, d1 = quantize_rows_groups(x, group=256)
    q0, s0, d0 = quantize_rows(x)
    assert np.array_equal(q1, q0) and np.array_equal(s1[:, 0], s0) and np.array_equal(d1[:, 0], d0)
    x[2, 128:] = 0.0
    q, s, d = quantize_rows_groups(x)
    assert s[2, 1] == 1.0 and d[2, 1] == 1.0 and not np.any(q[2, 128:])
    w = round_bf16(rng.standard_normal((256, 24))).astype(np.float32)
    qw, sw, dw = quantize_columns_groups(w)
    assert sw.shape == (2, 24)
    for b in range(2):   # a block of rows per column is that column's per-column rule
        qb, sb, db = quantize_columns(w[b * GROUP:(b + 1) * GROUP])
        assert np.array_equal(qw[b * GROUP:(b + 1) * GROUP], qb) and np.array_equal(sw[b], sb)


def test_group_up_projection_equals_bf16_when_quantisation_is_exact():
    """Entries +-2^j whose group (token) or block (weight column) maximum is a power of two
    quantise exactly: scale = 448 / 2^m and the codes are 448 * 2^(j - m), exact in E4M3.
    The descaled group sums then equal x . W1 up to the float32 rounding of the descales, so
    the per-group and bf16 up-projections agree to ~1e-6.  Group maxima differ from group to
    group and from row to row, so a scale applied to the wrong group would show."""
    rng = np.random.default_rng(13)
    T, H, I, E, K = 6, 256, 8, 2, 2
    ng = H // GROUP
    gmax = np.exp2(-rng.integers(0, 5, (T, ng)))
    x = np.where(rng.random((T, H)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (T, H)) * gmax.repeat(GROUP, 1)
    x[:, 0::GROUP] = gmax
    bmax = np.exp2(-rng.integers(0, 5, (E, ng, 2 * I)))
    W1 = np.where(rng.random((E, H, 2 * I)) < 0.5, -1.0, 1.0) * 2.0 ** -rng.integers(0, 4, (E, H, 2 * I))
    W1 = W1 * bmax.repeat(GROUP, 1)
    W1[:, 0::GROUP, :] = bmax
    W2 = rng.standard_normal((E, I, H))
    ids = np.array([[0, 1]] * T)
    w = np.full((T, K), 0.5, np.float32)
    mg = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="group")
    m16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")
    for e in range(E):
        hg, h16 = mg.up(e, x), m16.up(e, x)
        assert np.allclose(hg, h16, rtol=1e-6, atol=1e-9 * np.abs(h16).max())
    q, s, d = quantize_rows_groups(x)   # the codes carry x exactly, up to the float32 descale
    assert np.allclose(q * d.astype(np.float64).repeat(GROUP, 1), x, rtol=2e-7, atol=0)


def test_group_up_projection_error_is_bounded():
    """Generic data: each E4M3 code has relative error <= 2^-4 of its group's scaled value
    (2^-10 of the group maximum below the normal range), so h moves by a bounded amount;
    groups of very different magnitude are not dragged down to the largest one."""
    rng = np.random.default_rng(14)
    T, H, I, E, K = 8, 384, 16, 3, 2
    x = round_bf16(rng.standard_normal((T, H)) * np.exp2(rng.integers(-8, 8, (T, H // GROUP))).repeat(GROUP, 1))
    W1 = round_bf16(rng.standard_normal((E, H, 2 * I)) / 8)
    W2 = round_bf16(rng.standard_normal((E, I, H)) / 4)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    w = np.full((T, K), 0.5, np.float32)
    mg = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="group")
    m16 = MoEFFN(x, ids, w, W1, W2, mode="pure", gmm1="bf16")

    def dev(v, gmax):
        return 2.0 ** -4 * np.abs(v) + gmax * 2.0 ** -18

    gx = np.abs(x).reshape(T, -1, GROUP).max(axis=2).repeat(GROUP, 1)
    dx = dev(x, gx)
    for e in range(E):
        gw = np.abs(W1[e]).reshape(-1, GROUP, 2 * I).max(axis=1).repeat(GROUP, 0)
        dw = dev(W1[e], gw)
        bound = dx @ (np.abs(W1[e]) + dw) + np.abs(x) @ dw
        assert np.all(np.abs(mg.up(e, x) - m16.up(e, x)) <= bound * (1 + 1e-6))


def test_scale_clamped_where_448_over_max_overflows():
    """A row whose largest value is ~1e-38 (a bf16 subnormal range value): 448 / max
    overflows float32; the scale is the largest finite float32, the codes stay finite
    and equal torch's E4M3 cast of x * FLT_MAX, and zeros stay zero."""
    import torch
    x = np.zeros((2, 64), np.float32)
    x[0, ::3] = np.float32(1e-38) * np.linspace(-1, 1, 22).astype(np.float32)
    x[1, 5] = np.float32(9.2e-41)                      # the smallest bf16 subnormal magnitude
    x = round_bf16(x).astype(np.float32)
    q, scale, descale = quantize_rows(x)
    fmax = np.finfo(np.float32).max
    assert np.all(scale == fmax) and np.all(np.isfinite(q))
    ref = (torch.tensor(x) * torch.tensor(fmax)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(q, ref)
    assert np.all(q[x == 0] == 0)
    assert np.all(descale == np.float32(1.0) / fmax) and np.all(descale > 0)


# ------------------------------------------------ deviation bound of the row quantiser
def _torch_rows(v):
    """Per-row E4M3 quantisation with torch float32 ops and torch's float8 cast: (codes, descale)."""
    t = torch.tensor(np.asarray(v, np.float32))
    amax = t.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, torch.tensor(448.0) / amax, torch.ones_like(amax))
    scale = torch.minimum(scale, torch.tensor(np.finfo(np.float32).max))
    q = (t * scale).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return q, (1.0 / scale).to(torch.float64).numpy()[..., 0]


def test_quantize_rows_dev_covers_every_sampled_admissible_row():
    """Rows of bf16 values, some elements with an open decision of one bf16 ulp (the
    row maximum open in some rows): every admissible row (each element one of the bf16
    values within its deviation) quantises to codes within dq and a descale within rel."""
    from oracle.quant import quantize_rows_dev
    rng = np.random.default_rng(11)
    n, L = 24, 96
    v = round_bf16(rng.standard_normal((n, L)) * np.exp2(rng.integers(-3, 4, (n, 1))))
    ulp = np.exp2(np.floor(np.log2(np.abs(v) + 1e-300)) - 7)
    d = np.where(rng.random((n, L)) < 0.3, ulp, 0.0)
    d[::3, np.argmax(np.abs(v[::3]), axis=1)] = ulp[::3, np.argmax(np.abs(v[::3]), axis=1)]   # open row maxima
    dq, rel = quantize_rows_dev(v, d)
    q0, ds0 = _torch_rows(v)
    assert (dq > 0).any() and (rel > 0).any()
    worst_q = np.zeros_like(dq)
    worst_r = np.zeros(n)
    for _ in range(300):
        vp = v + d * rng.integers(-1, 2, (n, L))                   # each element: its value or a neighbour
        q, ds = _torch_rows(vp)
        worst_q = np.maximum(worst_q, np.abs(q - q0))
        worst_r = np.maximum(worst_r, np.abs(ds - ds0) / ds0)
    assert np.all(worst_q <= dq) and np.all(worst_r <= rel * (1 + 1e-12))
    assert (worst_q > 0).any()                                     # the check is not vacuous
    dq0, rel0 = quantize_rows_dev(v, np.zeros_like(v))
    assert not dq0.any() and not rel0.any()


def test_fp8_backward_act_grad_exact_when_rows_are_representable():
    """dY and W2 rows made of E4M3 values whose row maxima are 448 * 2^k: the per-row
    quantisation is exact, so the FP8 backward's G (seen through d_topk_weights and dH,
    hence dW1) equals the bf16 backward's in pure mode; dx still differs (dH rows are
    quantised) but stays within the E4M3 error of dH."""
    rng = np.random.default_rng(12)
    T, H, I, E, K = 24, 64, 64, 3, 2
    codes = round_e4m3(rng.uniform(-448, 448, (T + E * I, H)))
    codes[:, 0] = 448.0                                            # every row maximum is 448
    dY = codes[:T] * np.exp2(rng.integers(-9, -3, (T, 1)))
    W2 = (codes[T:] * np.exp2(rng.integers(-12, -8, (E * I, 1)))).reshape(E, I, H)
    x = round_bf16(rng.standard_normal((T, H)))
    W1 = round_bf16(rng.standard_normal((E, H, 2 * I)) / 8)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    w = rng.random((T, K)).astype(np.float32)
    a16 = MoEFFN(x, ids, w, W1, W2, dY=dY, mode="pure").backward()
    a8 = MoEFFN(x, ids, w, W1, W2, dY=dY, mode="pure", bwd="fp8").backward()
    np.testing.assert_allclose(a8[1], a16[1], rtol=1e-12, atol=1e-12)       # d_topk_weights
    np.testing.assert_allclose(a8[2], a16[2], rtol=1e-10, atol=1e-12)       # dW1 (from dH)
    np.testing.assert_allclose(a8[3], a16[3], rtol=1e-12, atol=1e-12)       # dW2 (dY, not quantised)
    err = np.abs(a8[0] - a16[0])
    assert err.max() > 0                                                   # dx: dH was quantised
    assert np.all(err <= 0.15 * np.abs(a16[0]).max())
