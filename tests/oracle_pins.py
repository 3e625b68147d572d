"""Checks that pin the CPU oracle to facts fixed by the pages and by mathematics.

Every check raises AssertionError on failure.  They are collected by
``test_oracle_pins.py`` and re-run against deliberately broken builds of the
oracle by ``test_oracle_mutants.py`` (a pin that no plausible mistake can
fail pins nothing).
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close_printed(value, printed, decimals):
    """value agrees with a number printed to `decimals` places."""
    return abs(float(value) - float(printed)) <= 0.5 * 10.0 ** (-decimals) + 1e-7


# --------------------------------------------------------------------------
# Worked examples printed on the pages.
# --------------------------------------------------------------------------
def check_six_weights():
    g = _golden("six_weights_int4.json")
    w = np.array(g["weights"], np.float32)
    q, s, z = oracle.asym_quantize(w, group=w.size, bits=g["bits"])
    assert abs(float(s[0, 0]) - g["scale"]) < 1e-7, s
    assert int(z[0, 0]) == g["zero_point"], z
    assert q[0].tolist() == g["codes"], q
    back = oracle.asym_dequantize(q, s, z, w.size)[0]
    for v, p in zip(back, g["recovered"]):
        assert _close_printed(v, p, g["recovered_printed_decimals"]), (v, p)
    err = np.abs(back.astype(np.float64) - w.astype(np.float64))
    assert _close_printed(err.max(), g["max_error"], 3), err
    assert err.max() <= g["half_step"] + 1e-7


def check_eight_weights():
    g = _golden("eight_weights_int4.json")
    w = np.array(g["weights"], np.float32)
    q, s, z = oracle.asym_quantize(w, group=w.size, bits=g["bits"])
    assert _close_printed(s[0, 0], g["scale"], g["scale_printed_decimals"]), s
    assert int(z[0, 0]) == g["zero_point"], z
    assert q[0].tolist() == g["codes"], q
    back = oracle.asym_dequantize(q, s, z, w.size)[0]
    for v, p in zip(back, g["back"]):
        assert _close_printed(v, p, g["back_printed_decimals"]), (v, p)
    assert _close_printed(back[-1], 0.468, 3)   # 0.47 -> 0.468


def check_int8_outlier():
    g = _golden("int8_outlier.json")
    base = np.array(g["group"], np.float32)
    q0, s0 = oracle.sym_quantize(base, base.size, 8)
    assert int(q0[0, 1]) == g["code_of_0p12_before"], q0
    with_outlier = np.append(base, np.float32(g["outlier"]))
    q1, s1 = oracle.sym_quantize(with_outlier, with_outlier.size, 8)
    ratio = float(s1[0, 0]) / float(s0[0, 0])
    assert abs(ratio - g["scale_ratio_after_over_before"]) < 1e-4, ratio
    assert int(q1[0, 0]) == g["code_of_0p04_after"], q1
    assert int(q1[0, 1]) == g["code_of_0p12_after"], q1
    back = oracle.sym_dequantize(q1, s1, with_outlier.size)[0]
    loss = 100.0 * (0.12 - float(back[1])) / 0.12
    assert abs(loss - g["loss_of_0p12_after_percent"]) < 1.0, loss


def check_int4_symmetric_exercise():
    g = _golden("int4_symmetric_exercise.json")
    x = np.array([g["absmax"], g["value"]], np.float32)
    q, s = oracle.sym_quantize(x, 2, 4)
    assert _close_printed(s[0, 0], g["step"], g["step_printed_decimals"]), s
    assert int(q[0, 1]) == g["code"]
    back = oracle.sym_dequantize(q, s, 2)[0]
    assert abs(abs(float(back[1]) - g["value"]) - g["error"]) < 1e-7
    assert int(q[0, 0]) == 7     # the largest magnitude maps to the largest code


def check_int4_outlier_slide():
    g = _golden("int4_outlier_slide.json")
    x = np.array(g["group"], np.float32)
    q, s = oracle.sym_quantize(x, x.size, 4)
    assert _close_printed(s[0, 0], g["step"], g["step_printed_decimals"]), s
    assert (q[0, :-1] == g["small_codes"]).all(), q
    assert int(q[0, -1]) == 7


# --------------------------------------------------------------------------
# Tie-breaking and the readings for degenerate groups.
# --------------------------------------------------------------------------
def check_round_half_even():
    # lo = 0, hi = 15 gives s = 1 and z = 0 exactly, so codes are rint(v).
    v = np.array([0.0, 15.0, 2.5, 3.5, 0.5, 1.5, 4.5, 14.5], np.float32)
    q, s, z = oracle.asym_quantize(v, group=v.size, bits=4)
    assert float(s[0, 0]) == 1.0 and int(z[0, 0]) == 0
    assert q[0].tolist() == [0, 15, 2, 4, 0, 2, 4, 14], q
    # INT8 row whose absmax is 127 has scale exactly 1.
    x = np.array([127.0, 2.5, -2.5, 0.5, -1.5], np.float32)
    qi, si = oracle.sym_quantize(x, x.size, 8)
    assert float(si[0, 0]) == 1.0
    assert qi[0].tolist() == [127, 2, -2, 0, -2], qi


def check_degenerate_groups():
    pos = np.linspace(0.1, 0.5, 8).astype(np.float32)
    q, s, z = oracle.asym_quantize(pos, group=8, bits=4)
    assert int(z[0, 0]) == 0 and q[0, -1] == 15
    assert abs(float(s[0, 0]) - np.float32(0.5) / np.float32(15)) == 0.0
    neg = -pos
    q, s, z = oracle.asym_quantize(neg, group=8, bits=4)
    assert int(z[0, 0]) == 15 and q[0, -1] == 0
    zero = np.zeros(8, np.float32)
    q, s, z = oracle.asym_quantize(zero, group=8, bits=4)
    assert float(s[0, 0]) == 1.0 and int(z[0, 0]) == 0 and (q == 0).all()
    back = oracle.asym_dequantize(q, s, z, 8)
    assert (back == 0).all()


# --------------------------------------------------------------------------
# Invariants the pages state, on seeded random groups.
# --------------------------------------------------------------------------
def _random_groups(n_groups=3000, group=128, seed=7):
    g = np.random.Generator(np.random.PCG64(seed))
    w = g.standard_normal((n_groups, group), dtype=np.float32) * np.float32(0.02)
    # a few groups with a large entry, a few with exact zeros, a few one-signed
    w[::17, 5] = np.float32(0.5)
    w[::13, 11] = 0.0
    w[::29] = np.abs(w[::29])
    w[::31] = -np.abs(w[::31])
    return w


def check_error_bound_and_zero():
    w = _random_groups()
    q, s, z = oracle.asym_quantize(w, group=w.shape[1], bits=4)
    back = oracle.asym_dequantize(q, s, z, w.shape[1])
    s64 = s.astype(np.float64)
    err = np.abs(back.astype(np.float64) - w.astype(np.float64))
    # rounding error at most half a step (plus fp32 rounding of w/s and (q-z)s)
    slack = 4 * np.spacing(np.abs(w).max(axis=1, keepdims=True).astype(np.float32)).astype(np.float64)
    assert (err <= s64 / 2 + slack).all(), float((err - s64 / 2).max())
    # zero maps to code z and back to exactly 0.0
    zmask = w == 0.0
    assert zmask.any()
    assert (back[zmask] == 0.0).all()
    zz = np.broadcast_to(z, q.shape)
    assert (q[zmask] == zz[zmask]).all()
    # codes and zero-points in range; min -> 0 and max -> 15 when the group straddles 0
    assert q.max() <= 15 and z.max() <= 15
    straddle = (w.min(axis=1) < 0) & (w.max(axis=1) > 0)
    rows = np.nonzero(straddle)[0]
    assert (q[rows, w[rows].argmin(axis=1)] == 0).all()
    assert (q[rows, w[rows].argmax(axis=1)] == 15).all()


def check_nearest_grid_point():
    w = _random_groups(n_groups=400)
    q, s, z = oracle.asym_quantize(w, group=w.shape[1], bits=4)
    levels = np.arange(16, dtype=np.float64)
    grid = (levels[None, :] - z.astype(np.float64)) * s.astype(np.float64)      # [groups, 16]
    d = np.abs(w.astype(np.float64)[:, :, None] - grid[:, None, :])             # [groups, 128, 16]
    best = d.min(axis=2)
    chosen = np.take_along_axis(d, q.astype(np.int64)[:, :, None], axis=2)[:, :, 0]
    tol = 8 * np.spacing(np.float32(1.0)) * s.astype(np.float64)
    assert (chosen <= best + tol).all(), float((chosen - best).max())


def check_granularity_special_cases():
    wl = workloads.WORKLOADS["llama7b"]
    w, _ = workloads.weight(wl, 0, shape=(64, 1024))
    w = w.float().numpy()
    # per channel: group == cols; per tensor: one row holding everything
    qc, sc, zc = oracle.asym_quantize(w, group=w.shape[1], bits=4)
    assert sc.shape == (64, 1)
    qt, st, zt = oracle.asym_quantize(w.reshape(1, -1), group=w.size, bits=4)
    assert st.shape == (1, 1)
    lo, hi = min(w.min(), 0.0), max(w.max(), 0.0)
    assert float(st[0, 0]) == float(np.float32(np.float32(hi) - np.float32(lo)) / np.float32(15))
    # the same routine with G = 128 is finer: its error is smaller (assertion
    # of the granularity comparison in "How quantization works")
    qg, sg, zg = oracle.asym_quantize(w, group=128, bits=4)

    def rel(q, s, z, g):
        b = oracle.asym_dequantize(q, s, z, g).astype(np.float64).reshape(w.shape)
        return np.linalg.norm(b - w) / np.linalg.norm(w)

    e_group = rel(qg, sg, zg, 128)
    e_chan = rel(qc, sc, zc, w.shape[1])
    e_tensor = rel(qt, st, zt, w.size)
    assert e_group < e_chan < e_tensor, (e_group, e_chan, e_tensor)
    # symmetric INT8: per channel beats per tensor
    q8c, s8c = oracle.sym_quantize(w, w.shape[1], 8)
    q8t, s8t = oracle.sym_quantize(w.reshape(1, -1), w.size, 8)
    e8c = np.linalg.norm(oracle.sym_dequantize(q8c, s8c, w.shape[1]) - w) / np.linalg.norm(w)
    e8t = np.linalg.norm(oracle.sym_dequantize(q8t, s8t, w.size).reshape(w.shape) - w) / np.linalg.norm(w)
    assert e8c < e8t


def check_packing():
    vals = np.arange(10, dtype=np.uint8).reshape(2, 5) + 3
    p = oracle.pack_nibbles(vals)
    assert p.shape == (2, 3)
    assert p[0].tolist() == [3 | (4 << 4), 5 | (6 << 4), 7]
    assert p[1].tolist() == [8 | (9 << 4), 10 | (11 << 4), 12]


def check_code_words():
    # Two runs of 8 codes, the second reversed; expected bytes written out by
    # hand from the stated layout (element 2i at bits 4i, 2i+1 at bits 16+4i).
    vals = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 14, 13, 12, 11, 10, 9, 0]], np.uint8)
    p = oracle.pack_codes(vals)
    assert p.shape == (1, 8)
    # run 1 -> word 0x86427531; run 2: even elements 15, 13, 11, 9 give bits
    # 0-15 = 0x9BDF, odd elements 14, 12, 10, 0 give bits 16-31 = 0x0ACE
    assert p[0].tolist() == [0x31, 0x75, 0x42, 0x86, 0xDF, 0x9B, 0xCE, 0x0A]
    # unpacking by the same rule returns the codes
    words = p.view("<u4").reshape(-1)
    back = [(int(w) >> (4 * (e // 2) + 16 * (e % 2))) & 0xF for w in words for e in range(8)]
    assert back == vals[0].tolist()


def check_storage_70b():
    g = _golden("storage_70b.json")
    n, k = 8, 1024
    codes, scales, zeros = oracle.quantize_groupwise_packed(np.zeros((n, k), np.float32))
    weights = n * k
    groups = weights // 128
    assert codes.nbytes == weights // 2 and zeros.nbytes == groups // 2
    # with the page's 16-bit scale: 0.5 + 2.5/128 bytes per parameter
    per_param = (codes.nbytes + zeros.nbytes + 2 * groups) / weights
    assert abs(per_param - (0.5 + 2.5 / 128)) < 1e-12
    assert abs(g["params"] * per_param / 1e9 - g["total_gb"]) < 0.05
    assert abs(100 * per_param / 2 - g["fraction_percent"]) < 0.5


# --------------------------------------------------------------------------
# Matmul references.
# --------------------------------------------------------------------------
def check_matmul_against_blas():
    g = np.random.Generator(np.random.PCG64(11))
    a = g.standard_normal((5, 67), dtype=np.float32)
    b = g.standard_normal((9, 67), dtype=np.float32)
    c = oracle.matmul_nt_f64(a, b)
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    assert c.shape == (5, 9)
    assert np.allclose(c, ref, rtol=1e-12, atol=1e-12)


def check_w4a16_integer_case():
    # s = 1 and z = 0 turn the W4A16 product into an integer matvec.
    g = np.random.Generator(np.random.PCG64(12))
    q = g.integers(0, 16, size=(7, 256)).astype(np.uint8)
    x = g.integers(-4, 5, size=(3, 256)).astype(np.float32)
    s = np.ones((7, 2), np.float32)
    z = np.zeros((7, 2), np.uint8)
    y = oracle.w4a16_reference(x, q, s, z, 128)
    ref = x.astype(np.int64) @ q.astype(np.int64).T
    assert (y == ref).all()
    # non-trivial zero-points shift by z * sum(x) per group
    z2 = g.integers(0, 16, size=(7, 2)).astype(np.uint8)
    y2 = oracle.w4a16_reference(x, q, s, z2, 128)
    zf = np.repeat(z2.astype(np.int64), 128, axis=1)
    ref2 = x.astype(np.int64) @ (q.astype(np.int64) - zf).T
    assert (y2 == ref2).all()


def check_int8_matmul():
    g = np.random.Generator(np.random.PCG64(13))
    a = g.integers(-128, 128, size=(6, 300)).astype(np.int8)
    b = g.integers(-128, 128, size=(4, 300)).astype(np.int8)
    acc = oracle.int8_matmul_nt(a, b)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert (acc == ref).all()
    y = oracle.rescale_f64(acc, np.float32([0.5, 2, 1, 1, 1, 0.25]), np.float32([1, 3, 1, 0.5]))
    assert y[1, 1] == ref[1, 1] * 6 and y[5, 3] == ref[5, 3] * 0.125


def check_smoothquant_invariants():
    wl = workloads.WORKLOADS["smoothquant"]
    x, cols = workloads.sq_activations(wl, 64, 512)
    w, _ = workloads.weight(wl, 0, shape=(96, 512))
    x = x.float().numpy()
    w = w.float().numpy()
    cx, cw = oracle.col_absmax(x), oracle.col_absmax(w)
    assert (cx == np.abs(x).max(axis=0)).all() and (cw == np.abs(w).max(axis=0)).all()
    s = oracle.smooth_factors(cx, cw, 0.5)
    # closed form: s_j^2 = cx_j / cw_j (alpha = 1/2)
    assert np.allclose(s.astype(np.float64) ** 2, cx.astype(np.float64) / cw.astype(np.float64), rtol=1e-6)
    xs = oracle.scale_columns_div(x, s)
    ws = oracle.scale_columns_mul(w, s)
    # alpha = 1/2 balances the channel maxima of the two operands
    assert np.allclose(oracle.col_absmax(xs), oracle.col_absmax(ws), rtol=1e-6)
    # the smoothing leaves the product unchanged (up to fp32 rounding of Xs, Ws)
    y = oracle.matmul_nt_f64(x, w)
    ys = oracle.matmul_nt_f64(xs, ws)
    assert np.linalg.norm(ys - y) / np.linalg.norm(y) < 1e-6
    # outlier channels get the largest smoothing factors
    assert set(np.argsort(s)[-len(cols):]) == set(cols.tolist())
    # floors: an all-zero activation channel gives sqrt(1e-5) / sqrt(cw)
    cx0 = cx.copy()
    cx0[0] = 0.0
    s0 = oracle.smooth_factors(cx0, cw, 0.5)
    assert abs(float(s0[0]) - np.sqrt(1e-5) / np.sqrt(float(cw[0]))) < 1e-6 * float(s0[0])


def _smooth_listing_columns():
    """Column maxima over nine decades, plus the floor cases: a weight column
    below the 1e-5 floor, an activation column below it, both below it, both
    zero, and each exactly at it."""
    g = np.random.Generator(np.random.PCG64(41))
    cx = (10.0 ** g.uniform(-7, 2.5, 4000)).astype(np.float32)
    cw = (10.0 ** g.uniform(-7, 0, 4000)).astype(np.float32)
    fl = np.float32(1e-5)
    cx[:6] = [np.float32(3.0), np.float32(2e-7), np.float32(4e-6), 0.0, fl, np.float32(0.5)]
    cw[:6] = [np.float32(1e-7), np.float32(0.02), np.float32(3e-6), 0.0, np.float32(0.1), fl]
    return cx, cw


def check_smooth_factors_listing():
    # "How quantization works", "Activation quantization and outliers": the
    # listing computes, on float32 tensors,
    #   s = clamp(max|X_j|, min=1e-5) ** alpha / clamp(max|W_j|, min=1e-5) ** (1 - alpha).
    # (1) alpha = 1/2, bit for bit against that expression evaluated in numpy
    # float32 (its ** 0.5 is the correctly rounded IEEE square root, its '/'
    # the correctly rounded division), each maximum floored first.  The set
    # holds columns where the one-root form fl32(sqrt(cx/cw)) rounds
    # differently, so the two-root order of the listing is what is pinned.
    cx, cw = _smooth_listing_columns()
    fl = np.float32(1e-5)
    xf, wf = np.maximum(cx, fl), np.maximum(cw, fl)
    listing = (xf ** np.float32(0.5)) / (wf ** np.float32(1.0 - 0.5))
    assert listing.dtype == np.float32
    # the square roots are the correctly rounded ones (fp64 root, one rounding)
    assert np.array_equal(xf ** np.float32(0.5), np.sqrt(xf.astype(np.float64)).astype(np.float32))
    s = oracle.smooth_factors(cx, cw, 0.5)
    assert np.array_equal(s.view(np.uint32), listing.view(np.uint32)), np.nonzero(s != listing)[0][:5]
    one_root = np.sqrt(xf / wf).astype(np.float32)
    assert (one_root != listing).sum() > 100
    # the floor cases by their closed values
    assert s[0] == np.float32(np.sqrt(np.float32(3.0))) / np.float32(np.sqrt(fl))
    assert s[3] == np.float32(1.0) and s[4] == np.float32(np.sqrt(fl)) / np.float32(np.sqrt(np.float32(0.1)))
    # (2) torch's CPU evaluation of the same listing (whose float32 square
    # root is within one ulp but not always correctly rounded) agrees to an ulp.
    import torch
    tx, tw = torch.from_numpy(cx), torch.from_numpy(cw)
    ts = (tx.clamp(min=1e-5) ** 0.5 / tw.clamp(min=1e-5) ** (1 - 0.5)).numpy()
    assert np.abs(ts.view(np.int32).astype(np.int64) - s.view(np.int32).astype(np.int64)).max() <= 2
    # (3) alpha = 3/4 (the powf branch) against the closed form
    # xf^0.75 / wf^0.25 in fp64 and against torch's float32 listing, each to
    # a few ulps.
    s75 = oracle.smooth_factors(cx, cw, 0.75)
    exact = xf.astype(np.float64) ** 0.75 / wf.astype(np.float64) ** 0.25
    assert (np.abs(s75.astype(np.float64) - exact) <= 4 * np.spacing(np.abs(s75)).astype(np.float64)).all()
    t75 = (tx.clamp(min=1e-5) ** 0.75 / tw.clamp(min=1e-5) ** (1 - 0.75)).numpy()
    assert np.abs(t75.view(np.int32).astype(np.int64) - s75.view(np.int32).astype(np.int64)).max() <= 4
    # s(3/4) / s(1/2) = (xf wf)^(1/4): larger exactly where xf wf > 1
    prod = xf.astype(np.float64) * wf.astype(np.float64)
    assert (s75[prod > 1.01] > s[prod > 1.01]).all() and (s75[prod < 0.99] < s[prod < 0.99]).all()


def check_smoothquant_error_ordering():
    # "How quantization works", activation-outlier experiment: weight-only INT8
    # error < SmoothQuant W8A8 error < plain W8A8 error.  The listing there
    # quantizes the activations with one scale per tensor; the per-token form
    # (the online path of the W8A8 GEMM) keeps the same ordering.
    wl = workloads.WORKLOADS["smoothquant"]
    x, _ = workloads.sq_activations(wl, 256, 1024)
    w, _ = workloads.weight(wl, 0, shape=(256, 1024))
    x = x.float().numpy()
    w = w.float().numpy()
    y = oracle.matmul_nt_f64(x, w)

    def rel(yq):
        return np.linalg.norm(yq - y) / np.linalg.norm(y)

    qw, b = oracle.sq_quantize_weight(w, None)
    wq = oracle.sym_dequantize(qw, b[:, None], w.shape[1])
    err_w8 = rel(oracle.matmul_nt_f64(x, wq))
    _, _, _, y_plain = oracle.sq_w8a8_reference(x, None, qw, b)
    s = oracle.smooth_factors(oracle.col_absmax(x), oracle.col_absmax(w), 0.5)
    qws, bs = oracle.sq_quantize_weight(w, s)
    _, _, _, y_sq = oracle.sq_w8a8_reference(x, s, qws, bs)
    err_plain, err_sq = rel(y_plain), rel(y_sq)
    assert err_w8 < err_sq < err_plain, (err_w8, err_sq, err_plain)

    # the listing's own form: q8_per_tensor on the activations
    def per_tensor(xv, sv, qwv, bv):
        qx, a = oracle.sq_quantize_activation_per_tensor(xv, sv)
        return oracle.rescale_f64(oracle.int8_matmul_nt(qx, qwv), a, bv)

    err_plain_t = rel(per_tensor(x, None, qw, b))
    err_sq_t = rel(per_tensor(x, s, qws, bs))
    assert err_w8 < err_sq_t < err_plain_t, (err_w8, err_sq_t, err_plain_t)
    # the page reports SmoothQuant cutting the per-tensor W8A8 error to about a third
    assert err_sq_t < 0.5 * err_plain_t, (err_sq_t, err_plain_t)


def check_sym_error_bound():
    g = np.random.Generator(np.random.PCG64(14))
    x = g.standard_normal((50, 256), dtype=np.float32)
    q, s = oracle.sym_quantize(x, 256, 8)
    back = oracle.sym_dequantize(q, s, 256)
    err = np.abs(back.astype(np.float64) - x)
    assert (err <= s.astype(np.float64) / 2 * (1 + 1e-6) + 1e-7).all()
    assert (np.abs(q).max(axis=1) == 127).all()


def check_sym_zero_row_floor():
    # An all-zero row: the absmax is floored at 1e-8 before the division
    # (fake-quantization listing of "How quantization works"), so the scale is
    # finite and every code is 0.
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = 1.0
    q, s = oracle.sym_quantize(x, 64, 8)
    assert float(s[0, 0]) == float(np.float32(1e-8) / np.float32(127))
    assert (q[0] == 0).all() and int(q[1, 3]) == 127
    assert (oracle.sym_dequantize(q, s, 64)[0] == 0).all()


def check_sym_int4_stored_groups():
    # Symmetric INT4 per group of 128 in the stored format: the scale is the
    # closed form fl32(max(max|w|, 1e-8) / 7), every code is q + 8 with q in
    # [-7, 7] (|w/s| <= 7, so nothing is clipped and the extra level -8 is
    # unused), the group's largest magnitude maps to +-7, zero maps to code 8
    # and back to exactly 0, the error is at most half a step, each code is
    # the nearest of the 16 grid points, and every zero-point nibble is 8.
    w = _random_groups(n_groups=600)
    w[5] = 0.0                                          # an all-zero group
    codes, s, zeros, q = oracle.sym_quantize_int4_packed(w.reshape(300, 256), 128)
    codes, s, zeros, q = codes.reshape(600, 64), s.reshape(600, 1), zeros, q.reshape(600, 128)
    amax = np.abs(w).max(axis=1)
    expect = np.maximum(amax, np.float32(1e-8)).astype(np.float32) / np.float32(7)
    assert np.array_equal(s[:, 0], expect)
    assert q.min() >= -7 and q.max() <= 7
    big = np.abs(w).argmax(axis=1)
    rows = np.nonzero(amax > 0)[0]
    assert (np.abs(q[rows, big[rows]]) == 7).all()
    assert (q[w == 0.0] == 0).all() and (q[5] == 0).all()
    # storage: low/high nibbles of the code words hold q + 8 (layout as the
    # asymmetric codes), zero-points all 8
    unpacked = np.empty(q.shape, np.int16)
    words = codes.view(np.uint32)
    for i in range(8):
        nib = (i >> 1) + ((i & 1) << 2)
        unpacked[:, i::8] = (words >> np.uint32(4 * nib)) & np.uint32(15)
    assert np.array_equal(unpacked, q.astype(np.int16) + 8)
    assert zeros.shape == (300, 1) and (zeros == 0x88).all()
    # an odd group count leaves the last byte's high nibble as padding (0)
    assert (oracle.sym_quantize_int4_packed(w[:4].reshape(4, 128), 128)[2] == 0x08).all()
    back = (q.astype(np.float64)) * s.astype(np.float64)
    err = np.abs(back - w.astype(np.float64))
    assert (err <= s.astype(np.float64) / 2 * (1 + 1e-6) + 1e-12).all()
    grid = np.arange(-8, 8, dtype=np.float64)[None, None, :] * s.astype(np.float64)[:, :, None]
    d = np.abs(w.astype(np.float64)[:, :, None] - grid)
    chosen = np.take_along_axis(d, (q.astype(np.int64) + 8)[:, :, None], axis=2)[:, :, 0]
    assert (chosen <= d.min(axis=2) + 8 * np.spacing(np.float32(1.0)) * s.astype(np.float64)).all()


def check_per_tensor_activation():
    # Per-tensor INT8 activations against the (pinned) per-token form:
    # fl32(m / 127) is monotonic in m, so the tensor's scale is the largest
    # per-token scale; with equal row maxima the two forms agree exactly; and
    # one outlier row sets the tensor's scale and coarsens every other row,
    # so the per-tensor error exceeds the per-token error ("Activation
    # quantization and outliers").
    g = np.random.Generator(np.random.PCG64(21))
    x = g.standard_normal((64, 256)).astype(np.float32)
    sm = (g.random(256) + 0.5).astype(np.float32)
    qt, at = oracle.sq_quantize_activation_per_tensor(x, sm)
    qr, ar = oracle.sq_quantize_activation(x, sm)
    assert (at == ar.max()).all()
    xe = x.copy()
    xe[:, 0] = np.float32(100.0)                    # every row's absmax is column 0 after smoothing
    xe[:, 0] *= sm[0]
    qt2, at2 = oracle.sq_quantize_activation_per_tensor(xe, sm)
    qr2, ar2 = oracle.sq_quantize_activation(xe, sm)
    assert np.array_equal(at2, ar2) and np.array_equal(qt2, qr2)
    xo = x.copy()
    xo[7] *= np.float32(50.0)                       # an outlier token
    xs = oracle.scale_columns_div(xo, sm).astype(np.float64)
    qt3, at3 = oracle.sq_quantize_activation_per_tensor(xo, sm)
    qr3, ar3 = oracle.sq_quantize_activation(xo, sm)
    others = np.arange(64) != 7
    et = np.abs(qt3 * at3[:, None].astype(np.float64) - xs)[others].mean()
    er = np.abs(qr3 * ar3[:, None].astype(np.float64) - xs)[others].mean()
    assert et > 5 * er, (et, er)


def check_w8a16_reference():
    # Weight-only INT8 matmul ("How quantization works", "Mainstream schemes
    # at a glance", W8A16 row).  (1) Brute force on small integers with
    # power-of-two scales, where every product and sum is exact: distinct
    # shapes for tokens, rows and K and a distinct scale per row catch a
    # transposed operand or a scale taken from the wrong index.  (2) The
    # rounding bound of the pinned per-channel quantizer: each weight moves by
    # at most half its row's step, so |y - x W^T| <= b[n]/2 * sum_k |x[t, k]|.
    g = np.random.Generator(np.random.PCG64(31))
    T, N, K = 3, 5, 7
    x = g.integers(-9, 10, (T, K))
    q = g.integers(-128, 128, (N, K))
    b = np.array([2.0 ** -e for e in range(N)])
    y = oracle.w8a16_reference(x.astype(np.float32), q.astype(np.int8), b.astype(np.float32))
    for t in range(T):
        for n in range(N):
            exact = sum(int(x[t, k]) * int(q[n, k]) for k in range(K)) * b[n]
            assert y[t, n] == exact, (t, n, y[t, n], exact)
    w = (g.standard_normal((48, 320)) * np.linspace(0.1, 3.0, 48)[:, None]).astype(np.float32)
    xs = g.standard_normal((4, 320)).astype(np.float32)
    qw, bw = oracle.sq_quantize_weight(w, None)
    yq = oracle.w8a16_reference(xs, qw, bw)
    yr = xs.astype(np.float64) @ w.astype(np.float64).T
    bound = 0.5 * bw.astype(np.float64)[None, :] * np.abs(xs.astype(np.float64)).sum(1)[:, None]
    assert (np.abs(yq - yr) <= bound * (1 + 1e-6)).all()
    assert np.abs(yq - yr).max() > 0


# --------------------------------------------------------------------------
# Format variants: 16-bit scales, group sizes, 3- and 8-bit codes.
# --------------------------------------------------------------------------
def check_f16_conversion():
    # binary16 storage of scales ("How quantization works", Exercise 2: one
    # 16-bit scale per group).  Against numpy's IEEE conversion (round to
    # nearest even) on values over the whole range, on exact ties between
    # neighbours (normal and subnormal), and the saturation reading (R24):
    # at or above the largest finite value the result is 65504, not infinity.
    g = np.random.Generator(np.random.PCG64(51))
    a = (g.standard_normal(200000) * 10.0 ** g.uniform(-9, 4.8, 200000)).astype(np.float32)
    a = a[np.abs(a) < 65504]
    assert np.array_equal(oracle.f32_to_f16(a).view(np.uint16), a.astype(np.float16).view(np.uint16))
    # ties: halfway between consecutive binary16 values goes to the even one
    h = np.arange(1, 0x7BFF, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert (mid.astype(np.float64) == (lo + hi) / 2).all()
    got = oracle.f32_to_f16(mid).view(np.uint16)
    assert np.array_equal(got, np.where(h % 2 == 0, h, h + 1).astype(np.uint16))
    sat = oracle.f32_to_f16(np.float32([65504.0, 65519.0, 65520.0, 1e9, -1e9])).view(np.uint16)
    assert sat.tolist() == [0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF, 0xFBFF]
    assert oracle.f32_to_f16(np.float32([2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -24])).view(np.uint16).tolist() == [0, 2, 1]
    back = oracle.f16_to_f32(np.arange(0, 0x7C00, dtype=np.uint16))
    assert np.array_equal(back, np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32))


def check_f16_scale_grid():
    # 16-bit scales: the stored scale is the binary16 value of the fp32 scale
    # (1 if that is 0), and the codes are computed with the stored value, so
    # dequantizing with what is stored rounds each weight to its nearest grid
    # point (unclipped weights within half a stored step) and requantizing
    # the dequantized weights returns the codes.
    w = _random_groups(n_groups=800)
    w[3] = 0.0
    w[4] = np.float32(1e-9) * np.sign(w[4])          # a range below binary16's smallest step
    for sym in (False, True):
        q, s, z = oracle.quantize_format(w, 128, 4, symmetric=sym, scale_f16=True)
        qf, sf, zf = oracle.quantize_format(w, 128, 4, symmetric=sym, scale_f16=False)
        s16 = sf.astype(np.float16).astype(np.float32)
        s16[s16 == 0] = 1.0
        assert np.array_equal(s, s16)
        assert float(s[3, 0]) == 1.0 and float(s[4, 0]) == 1.0
        back = oracle.asym_dequantize(q, s, z, 128).astype(np.float64)
        levels = np.arange(16, dtype=np.float64)
        grid = (levels[None, :] - z.astype(np.float64)) * s.astype(np.float64)
        d = np.abs(w.astype(np.float64)[:, :, None] - grid[:, None, :])
        chosen = np.take_along_axis(d, q.astype(np.int64)[:, :, None], axis=2)[:, :, 0]
        assert (chosen <= d.min(axis=2) + 8 * np.spacing(np.float32(1.0)) * s.astype(np.float64)).all()
        inner = (q > 0) & (q < 15)
        err = np.abs(back - w.astype(np.float64))
        assert (err[inner] <= (s.astype(np.float64) / 2 * (1 + 1e-6) + 1e-12).repeat(1, 1)[
            np.nonzero(inner)[0], 0]).all()
        q2 = np.clip(np.rint(back.astype(np.float32) / s) + z, 0, 15)
        assert np.array_equal(q2.astype(np.uint8), q)
        # the stored format: two bytes per scale
        codes, ss, zz = oracle.pack_format(q, s, z, 4, True)
        assert ss.dtype == np.float16 and np.array_equal(ss.astype(np.float32), s)
    # the page's 70B storage estimate is this format: 0.5 B of codes, a 16-bit
    # scale and a 4-bit zero-point per 128 weights
    gld = _golden("storage_70b.json")
    codes, ss, zz = oracle.quantize_format_packed(np.zeros((8, 1024), np.float32), 128, 4, False, True)
    per_param = (codes.nbytes + ss.nbytes + zz.nbytes) / (8 * 1024)
    assert abs(per_param - (0.5 + 2.5 / 128)) < 1e-12
    assert abs(gld["params"] * per_param / 1e9 - gld["total_gb"]) < 0.05


def check_group_size_sweep():
    # "Quantization Explained", "Measuring Your Own Error": on a random normal
    # matrix the error rises as groups grow (32, 64, 128, 1024), and one huge
    # value makes it jump; "The Cost of Small Groups": a 16-bit scale and a
    # 4-bit zero-point cost (16 + 4) / group bits per weight.
    g = np.random.Generator(np.random.PCG64(52))
    w = g.standard_normal((64, 4096)).astype(np.float32)
    mse = []
    for group in (32, 64, 128, 1024):
        q, s, z = oracle.quantize_format(w, group, 4)
        mse.append(float(np.mean((oracle.asym_dequantize(q, s, z, group) - w) ** 2)))
        codes, ss, zz = oracle.quantize_format_packed(w, group, 4, False, True)
        assert abs((codes.nbytes + ss.nbytes + zz.nbytes) * 8 / w.size - (4 + 20 / group)) < 1e-12
    assert mse[0] < mse[1] < mse[2] < mse[3], mse
    wo = w.copy()
    wo[5, 77] = np.float32(50.0)
    q, s, z = oracle.quantize_format(wo, 128, 4)
    group_err = np.mean((oracle.asym_dequantize(q, s, z, 128)[5, :128] - wo[5, :128]) ** 2)
    q, s, z = oracle.quantize_format(w, 128, 4)
    clean_err = np.mean((oracle.asym_dequantize(q, s, z, 128)[5, :128] - w[5, :128]) ** 2)
    assert group_err > 20 * clean_err, (group_err, clean_err)


def check_bit_width_errors():
    # "Quantization from Scratch", "Measured on two real layers": with
    # group-128 scales the output error at 8, 4 and 3 bits was 0.64%, 10.98%,
    # 23.31% (layer 12) and 0.63%, 10.64%, 22.62% (layer 22): ratios of about
    # 2.1 (3 vs 4 bits) and 17 (4 vs 8 bits), which is what a rounding error
    # proportional to the step (hi - lo) / (2^b - 1) predicts (15/7 and
    # 255/15).  The same ratios on Gaussian weights and inputs, asymmetric and
    # symmetric, with each code the nearest of the 2^b grid points.
    g = np.random.Generator(np.random.PCG64(53))
    w = (g.standard_normal((96, 1024)) * 0.02).astype(np.float32)
    x = g.standard_normal((64, 1024)).astype(np.float32)
    y = x.astype(np.float64) @ w.astype(np.float64).T
    for sym in (False, True):
        err = {}
        for bits in (3, 4, 8):
            q, s, z = oracle.quantize_format(w, 128, bits, symmetric=sym)
            assert q.max() <= 2 ** bits - 1
            wq = oracle.asym_dequantize(q, s, z, 128).astype(np.float64)
            err[bits] = np.linalg.norm(x.astype(np.float64) @ wq.T - y) / np.linalg.norm(y)
            levels = np.arange(2 ** bits, dtype=np.float64)
            grid = (levels[None, :] - z.reshape(-1, 1).astype(np.float64)) * s.reshape(-1, 1).astype(np.float64)
            wg = w.reshape(-1, 128).astype(np.float64)
            d = np.abs(wg[:, :, None] - grid[:, None, :])
            chosen = np.take_along_axis(d, q.reshape(-1, 128).astype(np.int64)[:, :, None], axis=2)[:, :, 0]
            # slack: the fp32 rounding of w / s (quotients up to 2^b)
            tol = 4 * np.spacing(np.abs(wg).astype(np.float32)).astype(np.float64) + \
                8 * np.spacing(np.float32(1.0)) * s.reshape(-1, 1)
            assert (chosen <= d.min(axis=2) + tol).all()
        assert 1.8 < err[3] / err[4] < 2.5, err
        assert 13.0 < err[4] / err[8] < 21.0, err
        if not sym:
            assert 0.05 < err[4] < 0.2 and err[8] < 0.01, err


def check_codes3_packing():
    # 3-bit codes in the library's layout (consecutive codes 16 bits apart);
    # the expected words of one run of 32 codes written out by hand.
    vals = np.array([[1, 2, 3, 4, 5, 6, 7, 0] * 4], np.uint8)
    p = oracle.pack_codes3(vals)
    assert p.shape == (1, 12)
    # W0 holds elements 0..9: the even ones 1, 3, 5, 7, 1 at bits 0, 3, 6, 9,
    # 12 (0x1F59), the odd ones 2, 4, 6, 0, 2 at bits 16, 19, .. (0x21A2 << 16),
    # and bit 0 of element 30 (= 7) at bit 15; element 31 (= 0) adds nothing.
    # W1: 3, 5, 7, 1, 3 -> 0x33EB; 4, 6, 0, 2, 4 -> 0x4434.  W2: 5, 7, 1, 3, 5
    # -> 0x567D; 6, 0, 2, 4, 6 -> 0x6886.
    assert p.view("<u4")[0].tolist() == [0x21A29F59, 0x4434B3EB, 0x6886D67D]
    v2 = np.zeros((1, 32), np.uint8)
    v2[0, 30] = 6          # 0b110: bit 15 of W1 and W2
    v2[0, 31] = 3          # 0b011: bit 31 of W0 and W1
    assert oracle.pack_codes3(v2).view("<u4")[0].tolist() == [0x80000000, 0x80008000, 0x00008000]
    v3 = np.zeros((2, 64), np.uint8)
    v3[1, 32 + 13] = 7     # second row, second run: element 13 -> W1 bits 19..21
    w3 = oracle.pack_codes3(v3).view("<u4")
    assert w3.shape == (2, 6) and w3[1].tolist() == [0, 0, 0, 0, 0x00380000, 0] and not w3[0].any()


def check_symmetric_format():
    # The symmetric grid in the stored format (R22) is the pinned symmetric
    # quantizer ("How quantization works", "The math of quantization") shifted
    # by 2^(b-1): same scale, code q + 2^(b-1), zero-point 2^(b-1), so the
    # dequantized value (code - z) s is exactly q s.
    w = _random_groups(n_groups=300)
    w[7] = 0.0
    for bits in (3, 4, 8):
        q, s = oracle.sym_quantize(w, 128, bits, 1e-8)
        c, sf, zf = oracle.quantize_format(w, 128, bits, symmetric=True)
        assert np.array_equal(sf, s)
        assert (zf == 2 ** (bits - 1)).all()
        assert np.array_equal(c.astype(np.int16), q.astype(np.int16) + 2 ** (bits - 1))
        back = oracle.asym_dequantize(c, sf, zf, 128)
        assert np.array_equal(back, oracle.sym_dequantize(q, s, 128))


# --------------------------------------------------------------------------
# FP8 E4M3.
# --------------------------------------------------------------------------
def check_e4m3_conversion():
    # OCP E4M3 ("E4M3FN"): against torch's own float8_e4m3fn (an independent
    # implementation) on every code's value and on fp32 inputs over the whole
    # range below 464 (the midpoint above 448, beyond which rounding would
    # leave the finite values), including every exact tie between neighbours;
    # then the definition's landmarks and the saturation reading (R25).
    import torch
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle.from_e4m3(codes)
    tdec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    finite = ~np.isnan(tdec)
    assert np.array_equal(np.isnan(dec), ~finite) and np.array_equal(dec[finite], tdec[finite])
    g = np.random.Generator(np.random.PCG64(61))
    x = (g.standard_normal(400000) * 10.0 ** g.uniform(-4, 2.7, 400000)).astype(np.float32)
    x = x[np.abs(x) < 464]
    mids = ((dec[:-1].astype(np.float64) + dec[1:].astype(np.float64)) / 2)
    mids = mids[np.isfinite(mids) & (np.abs(mids) < 464)].astype(np.float32)
    for v in (x, mids, -mids):
        assert np.array_equal(oracle.to_e4m3(v), torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert float(oracle.from_e4m3(np.uint8([0x7E]))[0]) == 448.0           # largest finite
    assert float(oracle.from_e4m3(np.uint8([0x08]))[0]) == 2.0 ** -6       # smallest normal
    assert float(oracle.from_e4m3(np.uint8([0x01]))[0]) == 2.0 ** -9       # smallest subnormal
    assert float(oracle.from_e4m3(np.uint8([0x38]))[0]) == 1.0             # exponent bias 7
    assert oracle.to_e4m3(np.float32([448.0, 460.0, 464.0, 500.0, 1e6, -1e6])).tolist() == [0x7E] * 5 + [0xFE]


def check_fp8_listing():
    # "How quantization works", fake-quantization listing: s = max|w| / 448,
    # q = E4M3(w / s); the largest magnitude maps to +-448 exactly, every
    # weight in E4M3's normal range is within half an E4M3 step (2^-4
    # relative) of its value, and the page's error ordering on a weight
    # matrix: INT8 per channel < FP8 per tensor < INT8 per tensor (its table:
    # 0.0097 < 0.0265 < 0.0362).
    w, _ = workloads.weight(workloads.WORKLOADS["mlp70b"], 0, shape=(512, 2048))
    w = w.float().numpy()
    q, s = oracle.fp8_quantize(w, per_tensor=True)
    amax = np.float32(np.abs(w).max())
    assert (s == amax / np.float32(448.0)).all()
    back = oracle.from_e4m3(q).astype(np.float64) * np.float64(s[0])
    i = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert abs(float(oracle.from_e4m3(np.uint8([q[i]]))[0])) == 448.0
    xs = np.abs(w.astype(np.float64)) / np.float64(s[0])
    normal = xs >= 2.0 ** -6
    err = np.abs(back - w.astype(np.float64))
    assert (err[normal] <= 2.0 ** -4 * np.abs(w.astype(np.float64))[normal] * (1 + 1e-6) + 1e-30).all()
    assert (err[~normal] <= 2.0 ** -10 * np.float64(s[0]) * (1 + 1e-6)).all()

    def rel(a):
        return np.linalg.norm(a - w.astype(np.float64)) / np.linalg.norm(w.astype(np.float64))

    e_fp8 = rel(back)
    qt, st = oracle.sym_quantize(w.reshape(1, -1), w.size, 8)
    e_i8t = rel(oracle.sym_dequantize(qt, st, w.size).reshape(w.shape))
    qc, sc = oracle.sym_quantize(w, w.shape[1], 8)
    e_i8c = rel(oracle.sym_dequantize(qc, sc, w.shape[1]))
    assert e_i8c < e_fp8 < e_i8t, (e_i8c, e_fp8, e_i8t)
    # per row: one scale per row, each row's largest magnitude at +-448
    qr, sr = oracle.fp8_quantize(w)
    assert np.array_equal(sr, (np.abs(w).max(axis=1) / np.float32(448.0)).astype(np.float32))
    assert (np.abs(oracle.from_e4m3(qr)).max(axis=1) == 448.0).all()


def check_fp8_product():
    # The FP8 product reference: brute force on codes whose values are small
    # integers and powers of two (every product and sum exact), with distinct
    # shapes so a transposed operand or a wrong index fails; and the online
    # W8A8 reference against the dequantized product.
    g = np.random.Generator(np.random.PCG64(62))
    vals = np.float32([0, 1, -1, 2, -3, 0.5, 4, -0.25, 7, 12, -16])
    a = vals[g.integers(0, len(vals), (3, 40))]
    b = vals[g.integers(0, len(vals), (5, 40))]
    qa, qb = oracle.to_e4m3(a), oracle.to_e4m3(b)
    assert np.array_equal(oracle.from_e4m3(qa), a) and np.array_equal(oracle.from_e4m3(qb), b)
    acc = oracle.fp8_matmul_nt(qa, qb)
    for i in range(3):
        for j in range(5):
            assert acc[i, j] == sum(float(a[i, t]) * float(b[j, t]) for t in range(40))
    x = g.standard_normal((6, 64)).astype(np.float32)
    w = (g.standard_normal((7, 64)) * 0.05).astype(np.float32)
    qw, bw = oracle.fp8_quantize(w)
    qx, ax, y = oracle.fp8_w8a8_reference(x, qw, bw)
    xd = oracle.from_e4m3(qx).astype(np.float64) * ax.astype(np.float64)[:, None]
    wd = oracle.from_e4m3(qw).astype(np.float64) * bw.astype(np.float64)[:, None]
    assert np.allclose(y, xd @ wd.T, rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# LLM.int8(): "Quantization" (Engine Room ch. 15), "The Mathematics" and the
# history of LLM.int8(); "Quantization: Smaller Weights, Same Answers
# (Mostly)", the outlier families.
# --------------------------------------------------------------------------
def _w16(qw, b, x_dtype):
    """The 16-bit weights q * b (float32 product, one cast by torch)."""
    import torch
    wf = qw.astype(np.float32) * np.asarray(b, np.float32)[:, None]
    return torch.from_numpy(wf).to(torch.bfloat16 if x_dtype == "bf16" else torch.float16).float().numpy()


def _llm_case(seed, m=9, k=192, n=11, x_dtype="bf16"):
    g = np.random.Generator(np.random.PCG64(seed))
    x = workloads.gaussian(g, (m, k), 1.0)
    w = workloads.gaussian(g, (n, k), 0.05)
    x = workloads.to_dtype(x, x_dtype).float().numpy()
    qw, b = oracle.sq_quantize_weight(w, None)
    return x, qw, b


def check_llm_int8_special_cases():
    # no outlier dimension (threshold above every |x|): the plain vector-wise
    # INT8 product; every dimension an outlier: the plain 16-bit product of
    # the activations with the dequantized weights, the integer part empty
    for x_dtype in ("bf16", "f16"):
        x, qw, b = _llm_case(3, x_dtype=x_dtype)
        idx, found, qx, a, y = oracle.llm_int8_reference(x, qw, b, np.inf, x_dtype=x_dtype)
        qx0, a0, _, y0 = oracle.sq_w8a8_reference(x, None, qw, b)
        assert len(idx) == 0 and found == 0
        assert np.array_equal(qx, qx0) and np.array_equal(a, a0) and np.array_equal(y, y0)
        idx, found, qx, a, y = oracle.llm_int8_reference(x, qw, b, 0.0, x_dtype=x_dtype)
        assert idx.tolist() == list(range(x.shape[1])) and found == x.shape[1]
        assert not qx.any() and (a == np.float32(1e-8) / np.float32(127.0)).all()
        assert np.array_equal(y, oracle.matmul_nt_f64(x, _w16(qw, b, x_dtype)))


def check_llm_int8_decomposition():
    # C = S_out (X_q W_q) + X_16 W_16: outlier columns planted in some tokens
    # (one reaching the threshold exactly, one just below it, one in a
    # single token only), then the result against the vector-wise product of
    # the remaining columns plus the 16-bit product of the outlier ones
    for x_dtype in ("bf16", "f16"):
        x, qw, b = _llm_case(5, x_dtype=x_dtype)
        tau = 6.0
        x[:, 17] *= 40.0
        x[4, 60] = tau                                   # reaches the threshold: outlier
        x[:, 61] = np.clip(x[:, 61], -5.0, 5.0)
        x[2, 61] = 5.9375                                # just below it (exact in both types)
        x[:, 100] = np.clip(x[:, 100], -5.0, 5.0)
        x[7, 100] = -250.0                               # one token only, negative
        x[:, 150] *= 9.0
        cm = np.abs(x).max(axis=0)
        expect = np.nonzero(cm >= tau)[0]
        assert {17, 60, 100}.issubset(expect) and 61 not in expect
        idx, found, qx, a, y = oracle.llm_int8_reference(x, qw, b, tau, x_dtype=x_dtype)
        assert idx.tolist() == expect.tolist() and found == len(expect)
        xr = x.copy()
        xr[:, expect] = 0.0
        qx0, a0, _, y0 = oracle.sq_w8a8_reference(xr, None, qw, b)
        assert np.array_equal(qx, qx0) and np.array_equal(a, a0)
        # the largest-magnitude columns no longer set the token scales
        assert (a <= np.float32(np.abs(xr).max()) / np.float32(127.0) * (1 + 1e-6)).all()
        w16 = _w16(qw, b, x_dtype)
        yo = oracle.matmul_nt_f64(np.ascontiguousarray(x[:, expect]), np.ascontiguousarray(w16[:, expect]))
        assert np.array_equal(y, y0 + yo)


def check_llm_int8_cap_and_permutation():
    # a cap below the number found keeps the first columns in column order;
    # the rest stay in the integer product.  Permuting the feature order of
    # X and W together permutes X_q and leaves the product unchanged.
    x, qw, b = _llm_case(8, m=13, k=256, n=7)
    for c in (9, 40, 41, 200):
        x[3, c] = 30.0 + c
    idx, found, qx, a, y = oracle.llm_int8_reference(x, qw, b, 6.0, max_outliers=2)
    assert idx.tolist() == [9, 40] and found == 4
    xr = x.copy()
    xr[:, [9, 40]] = 0.0
    _, a0, _, y0 = oracle.sq_w8a8_reference(xr, None, qw, b)
    assert np.array_equal(a, a0)
    yo = oracle.matmul_nt_f64(np.ascontiguousarray(x[:, [9, 40]]), np.ascontiguousarray(_w16(qw, b, "bf16")[:, [9, 40]]))
    assert np.array_equal(y, y0 + yo)
    perm = np.random.Generator(np.random.PCG64(2)).permutation(x.shape[1])
    xp, qwp = np.ascontiguousarray(x[:, perm]), np.ascontiguousarray(qw[:, perm])
    _, full_found, qx1, a1, y1 = oracle.llm_int8_reference(x, qw, b, 6.0)
    idxp, foundp, qxp, ap, yp = oracle.llm_int8_reference(xp, qwp, b, 6.0)
    assert foundp == full_found == 4 and sorted(perm[idxp].tolist()) == [9, 40, 41, 200]
    assert np.array_equal(qxp, qx1[:, perm]) and np.array_equal(ap, a1)
    assert np.allclose(yp, y1, rtol=1e-12, atol=1e-12 * np.abs(y1).max())


def check_llm_int8_accuracy():
    # the pages' claim: carving the outlier dimensions out gives INT8
    # inference with the accuracy of the 16-bit activations.  On activations
    # with six outlier channels the planted channels are exactly the ones
    # found, the error stays within 10% of weight-only INT8 (activations
    # exact) and far below the vector-wise W8A8 product without the
    # carve-out, and more than 99.8% of the features go through INT8.
    wl = workloads.WORKLOADS["smoothquant"]
    x, cols = workloads.sq_activations(wl, 256, 1024)
    w, _ = workloads.weight(wl, 0, shape=(256, 1024))
    x = x.float().numpy()
    w = w.float().numpy()
    y = oracle.matmul_nt_f64(x, w)

    def rel(yq):
        return np.linalg.norm(yq - y) / np.linalg.norm(y)

    qw, b = oracle.sq_quantize_weight(w, None)
    err_w8 = rel(oracle.matmul_nt_f64(x, oracle.sym_dequantize(qw, b[:, None], w.shape[1])))
    _, _, _, y_plain = oracle.sq_w8a8_reference(x, None, qw, b)
    idx, found, _, _, y_llm = oracle.llm_int8_reference(x, qw, b, 6.0)
    assert idx.tolist() == sorted(int(c) for c in cols) and found == 6
    err_llm, err_plain = rel(y_llm), rel(y_plain)
    assert err_w8 < err_llm < 1.1 * err_w8, (err_w8, err_llm)
    assert err_llm < 0.2 * err_plain, (err_llm, err_plain)


def _awq_case(seed, n=48, k=256, t=40, salient=None):
    g = np.random.Generator(np.random.PCG64(seed))
    w = workloads.to_dtype(workloads.gaussian(g, (n, k), 0.02), "bf16").float().numpy()
    x = workloads.gaussian(g, (t, k), 1.0)
    if salient is not None:
        x[:, salient] *= np.float32(50.0)
    return w, workloads.to_dtype(x, "bf16").float().numpy()


def check_awq_alpha0_is_round_to_nearest():
    # alpha = 0 gives s = 1 in every channel: the codes are the plain
    # group-128 quantizer's and the error is ||X (W - W_hat)^T||^2 (here by
    # numpy's product of the dequantized weights).
    w, x = _awq_case(1)
    err, best, s, q, sc, z = oracle.awq_search_reference(w, x, alphas=[0.0])
    assert best == 0 and np.array_equal(s, np.ones_like(s))
    q0, s0, z0 = oracle.asym_quantize(w)
    assert np.array_equal(q, q0) and np.array_equal(sc.view(np.uint32), s0.view(np.uint32)) and np.array_equal(z, z0)
    w_hat = (q0.astype(np.float64) - np.repeat(z0, 128, axis=1)) * np.repeat(s0.astype(np.float64), 128, axis=1)
    d = x.astype(np.float64) @ (w.astype(np.float64) - w_hat).T
    assert np.isclose(err[0], np.sum(d * d), rtol=1e-6)


def check_awq_uniform_magnitudes():
    # every channel with the same mean |x|: s = 1 for every alpha, all errors
    # equal, and the first alpha is kept -- no channel to protect, nothing to
    # gain (the pages: the scaling helps where there are outliers, only there)
    w, _ = _awq_case(2)
    signs = np.where(np.random.Generator(np.random.PCG64(3)).random((40, 256)) < 0.5, -1.0, 1.0)
    x = (signs * 0.75).astype(np.float32)
    err, best, s, _, _, _ = oracle.awq_search_reference(w, x)
    assert best == 0 and np.all(err == err[0]) and np.array_equal(s, np.ones_like(s))


def check_awq_salient_channel():
    # one input channel 50x larger than the rest: some alpha > 0 cuts the
    # calibration output error ([QS] "Measured on two real layers": the
    # scaling helps the layer with large activation outliers)
    w, x = _awq_case(4, salient=17)
    err, best, s, _, _, _ = oracle.awq_search_reference(w, x)
    assert best > 0 and err[best] < 0.7 * err[0], (best, err)
    assert s[17] == s.max()          # the salient channel gets the largest factor


def check_awq_scales_closed_form():
    # channel j has mean |x| = j + 1 (j < 64: +-(j+1) over two tokens; from
    # 64 on: 2(j+1) and 0, so the mean and the largest value disagree):
    # alpha = 1 gives s_j = (j+1) / sqrt(128 * 1), alpha = 1/2 gives
    # sqrt(j+1) / 128^(1/4).
    k = 128
    j = np.arange(k, dtype=np.float64)
    x = np.zeros((2, k), np.float32)
    x[0, :64], x[1, :64] = j[:64] + 1, -(j[:64] + 1)
    x[0, 64:] = 2 * (j[64:] + 1)
    w, _ = _awq_case(5, n=16, k=k, t=2)
    _, _, s1, _, _, _ = oracle.awq_search_reference(w, x, alphas=[1.0])
    assert np.array_equal(s1, ((j + 1) / np.sqrt(128.0)).astype(np.float32))
    _, _, s2, _, _, _ = oracle.awq_search_reference(w, x, alphas=[0.5])
    want = (np.sqrt(j + 1) / 128.0 ** 0.25).astype(np.float32)
    assert np.all(np.abs(s2.view(np.int32) - want.view(np.int32)) <= 1)


def check_awq_factors_entry():
    # the factors-only entry gives every alpha's factors: the searched alpha's
    # row is the search's s_best bit for bit, and alpha = 0 is all ones
    w, x = _awq_case(10, salient=9)
    err, best, s, _, _, _ = oracle.awq_search_reference(w, x)
    s_all = oracle.awq_factors_reference(x)
    assert s_all.shape == (len(oracle.AWQ_ALPHAS), x.shape[1])
    assert np.array_equal(s_all[best].view(np.uint32), s.view(np.uint32))
    assert np.all(s_all[0] == 1.0)


def check_awq_power_of_two_invariance():
    # scaling the activations by 4 scales every magnitude alike: the same
    # factors and choice, the errors 16 times larger
    w, x = _awq_case(6, salient=3)
    e1, b1, s1, q1, _, _ = oracle.awq_search_reference(w, x)
    e4, b4, s4, q4, _, _ = oracle.awq_search_reference(w, 4.0 * x)
    assert b1 == b4 and np.allclose(s1, s4, rtol=2e-7, atol=0) and np.allclose(e4, 16.0 * e1, rtol=1e-9)


def check_awq_listing_error():
    # [QS]'s awq listing scores alpha by sum((D @ H) * D) with D = W - Q / s,
    # Q the round-to-nearest codes of W * s dequantized, and H from the
    # calibration inputs (here X^T X in fp64 by numpy): the same layer output
    # error ||X W^T - X diag(s)^-1 W_hat^T||^2.  The oracle folds diag(s)^-1
    # into the bf16 input instead (R32), which moves the error by the input's
    # rounding only (up to ~1e-3 of it here: the salient channel makes the
    # outputs large against their error); a wrong Q, a missing / s or another
    # H would move it by far more than the 1e-2 allowed.
    w, x = _awq_case(8, salient=11)
    h = x.astype(np.float64).T @ x.astype(np.float64)
    for alpha in (0.3, 0.7):
        err, _, s, q, sc, z = oracle.awq_search_reference(w, x, alphas=[alpha])
        w_hat = (q.astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(sc.astype(np.float64), 128, axis=1)
        d = w.astype(np.float64) - w_hat / s.astype(np.float64)[None, :]
        e = float(np.sum((d @ h) * d))
        assert abs(err[0] - e) <= 1e-2 * e, (alpha, err[0], e)


def check_awq_f16_input():
    # binary16 activations (R32: X / s rounded to the activations' own type):
    # at alpha = 0 nothing is rounded and the error is numpy's
    # ||X (W - W_hat)^T||^2 exactly as in bf16; at alpha = 1/2 the binary16
    # rounding (3 more bits than bf16) leaves the error closer to the
    # listing's unrounded sum((D H) * D) than the bf16 rounding does
    w, x = _awq_case(9, salient=5)
    x16 = workloads.to_dtype(x, "f16").float().numpy()
    err, best, s, q, sc, z = oracle.awq_search_reference(w, x16, alphas=[0.0], x_dtype="f16")
    w_hat = (q.astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(sc.astype(np.float64), 128, axis=1)
    d = x16.astype(np.float64) @ (w.astype(np.float64) - w_hat).T
    assert np.isclose(err[0], np.sum(d * d), rtol=1e-6)
    h = x16.astype(np.float64).T @ x16.astype(np.float64)
    e16, _, s, q, sc, z = oracle.awq_search_reference(w, x16, alphas=[0.5], x_dtype="f16")
    eb, _, sb, qb, _, _ = oracle.awq_search_reference(w, x16, alphas=[0.5], x_dtype="bf16")
    assert np.array_equal(s, sb) and np.array_equal(q, qb)      # the factors and codes do not depend on it
    w_hat = (q.astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(sc.astype(np.float64), 128, axis=1)
    dd = w.astype(np.float64) - w_hat / s.astype(np.float64)[None, :]
    e = float(np.sum((dd @ h) * dd))
    assert abs(e16[0] - e) < abs(eb[0] - e), (e16[0], eb[0], e)


ALL_CHECKS = [
    check_awq_alpha0_is_round_to_nearest, check_awq_uniform_magnitudes, check_awq_salient_channel,
    check_awq_scales_closed_form, check_awq_power_of_two_invariance, check_awq_listing_error, check_awq_f16_input,
    check_awq_factors_entry,
    check_llm_int8_special_cases, check_llm_int8_decomposition, check_llm_int8_cap_and_permutation,
    check_llm_int8_accuracy,
    check_e4m3_conversion, check_fp8_listing, check_fp8_product,
    check_symmetric_format,
    check_f16_conversion, check_f16_scale_grid, check_group_size_sweep, check_bit_width_errors,
    check_codes3_packing,
    check_per_tensor_activation,
    check_w8a16_reference,
    check_sym_int4_stored_groups,
    check_six_weights, check_eight_weights, check_int8_outlier, check_int4_symmetric_exercise,
    check_int4_outlier_slide, check_round_half_even, check_degenerate_groups, check_error_bound_and_zero,
    check_nearest_grid_point, check_granularity_special_cases, check_packing, check_code_words, check_storage_70b,
    check_matmul_against_blas, check_w4a16_integer_case, check_int8_matmul, check_smoothquant_invariants,
    check_smooth_factors_listing, check_smoothquant_error_ordering, check_sym_error_bound, check_sym_zero_row_floor,
]
