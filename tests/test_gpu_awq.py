"""GPU parity for AWQ's scaling search ("Quantization from Scratch", "AWQ:
protect the channels that matter"): the chosen factors and the INT4 codes,
scales and zero-points of W diag(s) bit for bit against the CPU oracle, every
alpha's calibration output error within the tolerance of its fp32-accumulated
products, and the chosen alpha the oracle's (or one whose oracle error ties
it within that tolerance).  Small ragged shapes, a salient channel, uniform
magnitudes (every alpha the same, so the first is kept), one alpha (plain
round-to-nearest), one calibration token, a reversed grid, binary16
activations (with X / s saturating at 65504), the 896 x 4864 layer shape of
the pages' measurements and the 4096 x 4096 layer with 2048 calibration
tokens."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import bits_equal, first_diff, note, stratified_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# err = sum_i (yref_i - yq_i)^2 over the T x N outputs, both products
# accumulated in fp32 on the GPU and in fp64 by the oracle.  Each GPU output
# carries an error delta_i of about sqrt(K) 2^-24 sum_k |x_k w_k| (a random
# walk of K roundings; both products: twice that, with a margin for the
# scaled and quantized operands), so err moves by 2 sum_i d_i delta_i +
# sum_i delta_i^2, d_i = yref_i - yq_i.  With the errors independent of d, the
# first sum stays within LAMBDA standard deviations, sqrt(err) * rms(delta).
# At the 4096-wide layer that is ~1e-5 of err; a single output (one token, one
# row) whose d cancels to almost nothing relies on it entirely.
LAMBDA = 6.0
U32 = 2.0 ** -24


def _err_tol(w, x, err_ref, rows=None):
    """Per-alpha tolerance on err (see above); rows: weight rows to estimate
    rms(sum_k |x_k w_k|) from (default all)."""
    wf = np.abs(w.float().numpy().astype(np.float64))
    if rows is not None:
        wf = wf[rows]
    xf = np.abs(x.float().numpy().astype(np.float64))
    k = xf.shape[1]
    beta = 2.5 * np.sqrt(k) * U32 * float(np.sqrt(np.mean((xf @ wf.T) ** 2)))
    outputs = x.shape[0] * w.shape[0]
    return 2 * LAMBDA * np.sqrt(np.asarray(err_ref)) * beta + outputs * beta ** 2 + 1e-12 * np.asarray(err_ref)


def _check_err(err, err_ref, w, x, what, rows=None):
    tol = _err_tol(w, x, err_ref, rows)
    bad = np.abs(err - err_ref) > tol
    assert not bad.any(), f"{what} err: got {err[bad]} want {np.asarray(err_ref)[bad]} tolerance {tol[bad]}"
    return tol


def _case(n, k, t, seed, salient=(), spread=None, dtype="bf16"):
    g = np.random.Generator(np.random.PCG64(seed))
    w = workloads.to_dtype(workloads.gaussian(g, (n, k), 0.02), dtype)
    x = workloads.gaussian(g, (t, k), 1.0)
    for c in salient:
        x[:, c] *= np.float32(50.0)
    if spread is not None:
        workloads.plant_scale_columns(x, g, max(1, k // 100), *spread)
    return w, workloads.to_dtype(x, dtype)


def _run(w, x, alphas, what):
    note(f"awq_search {what} W={tuple(w.shape)} X={tuple(x.shape)} alphas={len(alphas)}")
    codes, scales, zeros, smooth, err, best = qmm.awq_search(w.to(DEV), x.to(DEV), alphas)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy(), smooth.cpu().numpy(),
            err.cpu().numpy(), int(best.cpu().item()))


def _check_format(w, smooth, codes, scales, zeros, what, rows=None):
    """codes / scales / zeros == the oracle's group-128 INT4 of fl32(W diag(smooth))."""
    wf = w.float().numpy()
    if rows is not None:
        wf, codes, scales, zeros = wf[rows], codes[rows], scales[rows], zeros[rows]
    rc, rs, rz = oracle.quantize_groupwise_packed(oracle.scale_columns_mul(wf, smooth))
    assert bits_equal(scales, rs), f"{what} scales: {first_diff(scales, rs)}"
    assert bits_equal(zeros, rz), f"{what} zeros: {first_diff(zeros, rz)}"
    assert bits_equal(codes, rc), f"{what} codes: {first_diff(codes, rc)}"


def _xdt(x):
    return "f16" if x.dtype == torch.float16 else "bf16"


def _check(w, x, alphas, what, parallel=False, err_rtol=None):
    codes, scales, zeros, smooth, err, best = _run(w, x, alphas, what)
    xf = x.float().numpy()
    rerr, rbest, rs, _, _, _ = oracle.awq_search_reference(w.float().numpy(), xf, alphas, parallel=parallel,
                                                           x_dtype=_xdt(x))
    assert best == int(np.argmin(err)), f"{what}: best {best} is not the first minimum of {err}"
    if err_rtol is None:
        tol = _check_err(err, rerr, w, x, what)
    else:
        assert np.all(np.isfinite(err)), f"{what}: err {err}"
        tol = err_rtol * np.abs(rerr)
        assert np.all(np.abs(err - rerr) <= tol), f"{what} err: got {err} want {rerr}"
    if best != rbest:   # a near tie: the GPU's choice must be as good within the tolerance
        assert rerr[best] <= rerr[rbest] + tol[best] + tol[rbest], (what, best, rbest, rerr)
    s_all = oracle.awq_factors_reference(xf, alphas)
    assert bits_equal(smooth, s_all[best]), f"{what} smooth: {first_diff(smooth, s_all[best])}"
    if best == rbest:
        assert bits_equal(smooth, rs)
    _check_format(w, smooth, codes, scales, zeros, what)
    return err, best


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n,k,t,seed", [(48, 256, 40, 1), (200, 640, 100, 2), (129, 1152, 67, 3), (1, 128, 1, 4)])
def test_awq_ragged_shapes(n, k, t, seed, dtype):
    w, x = _case(n, k, t, seed, spread=(4.0, 58.0), dtype=dtype)
    _check(w, x, list(qmm.AWQ_ALPHAS), f"ragged n={n} k={k} t={t} {dtype}")


def test_awq_f16_input_saturates():
    # binary16: X / s past 65504 saturates there (R32 with R24).  Channel 0
    # holds 60000 in every token (the largest magnitude), channel 1 +-0.001
    # (the smallest), channel 2 a single 65000 among 9000 tokens: at alpha = 1
    # its factor is mag_2 / sqrt(max * min) ~ 0.93, so 65000 / s ~ 70000.
    t, k = 9000, 128
    g = np.random.Generator(np.random.PCG64(11))
    w = workloads.to_dtype(workloads.gaussian(g, (16, k), 0.02), "f16")
    x = workloads.gaussian(g, (t, k), 1.0)
    x[:, 0] = np.float32(60000.0)
    x[:, 1] = np.where(g.random(t) < 0.5, -1.0, 1.0).astype(np.float32) * np.float32(0.001)
    x[:, 2] = 0.0
    x[17, 2] = np.float32(65000.0)
    x = workloads.to_dtype(x, "f16")
    s1 = oracle.awq_factors_reference(x.float().numpy(), [1.0])[0]
    assert 65000.0 / s1[2] > 65504.0
    # Factors, codes and choice bit for bit; the error finite (an infinite
    # X / s would make it inf or NaN) and within 1e-2: the one 65504 entry
    # times the binary16 products' offset of 1024 (the codes enter as 1024 + q,
    # the zero-point's share taken back from the row sum) puts ~6.8e7 into an
    # fp32 partial sum whose rounding (8 at that size) the group scale of ~20
    # then carries into that token's outputs, far past the bound derived for
    # ordinary activations.
    _check(w, x, [1.0, 0.5], "binary16 saturation", err_rtol=1e-2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_awq_salient_channel(dtype):
    w, x = _case(96, 384, 64, 5, salient=(17,), dtype=dtype)
    err, best = _check(w, x, list(qmm.AWQ_ALPHAS), f"salient channel 17 {dtype}")
    assert best > 0 and err[best] < err[0]


def test_awq_uniform_magnitudes_keeps_first_alpha():
    # every channel with mean |x| = 0.75: s = 1 for every alpha, so every
    # alpha computes the same thing and the first is kept
    w, _ = _case(64, 256, 32, 6)
    signs = np.where(np.random.Generator(np.random.PCG64(7)).random((32, 256)) < 0.5, -1.0, 1.0)
    x = workloads.to_dtype((signs * 0.75).astype(np.float32), "bf16")
    codes, scales, zeros, smooth, err, best = _run(w, x, list(qmm.AWQ_ALPHAS), "uniform magnitudes")
    assert best == 0 and np.all(err == err[0]) and np.all(smooth == 1.0)
    rerr, _, _, _, _, _ = oracle.awq_search_reference(w.float().numpy(), x.float().numpy())
    _check_err(err, rerr, w, x, "uniform magnitudes")
    _check_format(w, smooth, codes, scales, zeros, "uniform magnitudes")


def test_awq_single_alpha_zero_is_round_to_nearest():
    # alpha = 0: s = 1, the codes are the plain group-128 quantizer's
    w, x = _case(80, 512, 24, 8, spread=(4.0, 58.0))
    codes, scales, zeros, smooth, err, best = _run(w, x, [0.0], "alpha 0 only")
    assert best == 0 and np.all(smooth == 1.0)
    c0, s0, z0 = qmm.quantize_groupwise(w.to(DEV))
    assert bits_equal(codes, c0.cpu().numpy()) and bits_equal(scales, s0.cpu().numpy())
    assert bits_equal(zeros, z0.cpu().numpy())
    rerr, _, _, _, _, _ = oracle.awq_search_reference(w.float().numpy(), x.float().numpy(), [0.0])
    _check_err(err, rerr, w, x, "alpha 0 only")


def test_awq_reversed_grid():
    # the grid's order is the caller's: reversed, the same alpha is found at
    # the mirrored index (unless two alphas tie)
    w, x = _case(64, 256, 48, 9, salient=(3, 200))
    grid = list(qmm.AWQ_ALPHAS)
    err_f, best_f = _check(w, x, grid, "forward grid")
    err_r, best_r = _check(w, x, grid[::-1], "reversed grid")
    assert bits_equal(err_r[::-1].copy(), err_f)
    assert best_r == len(grid) - 1 - best_f or err_f[best_f] == err_f[len(grid) - 1 - best_r]


def test_awq_layer_4096():
    # the 4096 x 4096 layer with 2048 calibration tokens, 1% of the channels
    # scaled 4x..58x: the factors bit for bit, the whole format bit for bit,
    # and the oracle's error of the chosen alpha and of its neighbours on the
    # grid (the oracle's fp64 products over every alpha would take minutes)
    wl = workloads.WORKLOADS["awq"]
    n, k = wl.weights[0]
    t = wl.batches[0]
    w, _ = workloads.weight(wl)
    x, _ = workloads.sq_activations(wl, t, k, n_channels=k // 100, lo=4.0, hi=58.0)
    grid = list(qmm.AWQ_ALPHAS)
    codes, scales, zeros, smooth, err, best = _run(w, x, grid, "layer 4096x4096, 2048 tokens")
    assert best == int(np.argmin(err))
    xf = x.float().numpy()
    s_all = oracle.awq_factors_reference(xf, grid)
    assert bits_equal(smooth, s_all[best]), f"smooth: {first_diff(smooth, s_all[best])}"
    _check_format(w, smooth, codes, scales, zeros, "layer 4096")
    near = [i for i in (best - 1, best, best + 1) if 0 <= i < len(grid)]
    rerr, rbest, _, _, _, _ = oracle.awq_search_reference(w.float().numpy(), xf, [grid[i] for i in near],
                                                          parallel=True)
    tol = _check_err(err[near], rerr, w, x, "err near the chosen alpha", rows=stratified_rows(n, 64))
    assert rerr[near.index(best)] <= rerr.min() + 2 * tol.max(), (near, rerr)


def test_awq_qwen_layer_shape():
    # the shape of the MLP down projections "Quantization from Scratch"
    # measures AWQ on ("Measured on two real layers": 4864-wide inputs, 896
    # outputs), with 2048 calibration tokens and the pages' channel spread
    # (largest mean |x| ~58x the median)
    w, x = _case(896, 4864, 2048, 10, spread=(4.0, 58.0))
    _check(w, x, list(qmm.AWQ_ALPHAS), "896x4864, 2048 tokens", parallel=True)


def test_awq_workspace_reuse_and_determinism():
    # one caller workspace for two calls (the second smaller), against fresh
    # workspaces: every output bit for bit, so nothing leaks from one call
    # into the next and the sums are taken in a fixed order
    big_w, big_x = _case(160, 512, 90, 12, spread=(4.0, 58.0))
    small_w, small_x = _case(64, 256, 30, 13, salient=(7,))
    grid = list(qmm.AWQ_ALPHAS)
    need = qmm.awq_workspace_bytes(160, 512, 90, len(grid))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)   # stale contents
    note("awq_search shared workspace, two calls")
    first = qmm.awq_search(big_w.to(DEV), big_x.to(DEV), grid, workspace=ws)
    second = qmm.awq_search(small_w.to(DEV), small_x.to(DEV), grid, workspace=ws)
    fresh_first = qmm.awq_search(big_w.to(DEV), big_x.to(DEV), grid)
    fresh_second = qmm.awq_search(small_w.to(DEV), small_x.to(DEV), grid)
    torch.cuda.synchronize()
    for got, want, what in ((first, fresh_first, "first"), (second, fresh_second, "second")):
        for g_, w_, name in zip(got, want, ("codes", "scales", "zeros", "smooth", "err", "best")):
            a, b = g_.cpu().numpy(), w_.cpu().numpy()
            assert bits_equal(a, b), f"{what} call {name}: {first_diff(a, b)}"


def test_awq_many_alphas():
    # 64 alphas (the most a call takes; the selection sums four per
    # wavefront) in an irregular order, against the oracle
    w, x = _case(72, 384, 50, 14, spread=(4.0, 58.0))
    grid = list(np.random.Generator(np.random.PCG64(15)).random(64))
    _check(w, x, grid, "64 alphas")
