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


def check_smoothquant_error_ordering():
    # "How quantization works", activation-outlier experiment: weight-only INT8
    # error < SmoothQuant W8A8 error < plain W8A8 error.
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


ALL_CHECKS = [
    check_per_tensor_activation,
    check_w8a16_reference,
    check_sym_int4_stored_groups,
    check_six_weights, check_eight_weights, check_int8_outlier, check_int4_symmetric_exercise,
    check_int4_outlier_slide, check_round_half_even, check_degenerate_groups, check_error_bound_and_zero,
    check_nearest_grid_point, check_granularity_special_cases, check_packing, check_code_words, check_storage_70b,
    check_matmul_against_blas, check_w4a16_integer_case, check_int8_matmul, check_smoothquant_invariants,
    check_smoothquant_error_ordering, check_sym_error_bound, check_sym_zero_row_floor,
]
