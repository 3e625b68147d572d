"""GPU parity: SmoothQuant W8A8 against the oracle (codes and scales bit for bit,
int32 accumulators exact, rescaled outputs within the stated tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import stratified_rows, assert_close, bits_equal, first_diff, note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def sq_inputs(m, k, n, xdt="bf16", wdt="bf16", seed=0):
    wl = workloads.WORKLOADS["smoothquant"]
    if seed == 0 and (m, k, n) == (2048, 4096, 4096):
        x, _ = workloads.sq_activations(wl, m, k)
        w, _ = workloads.weight(wl, 0)
        return x.to(TDT[xdt]) if xdt != "bf16" else x, w.to(TDT[wdt]) if wdt != "bf16" else w
    x = workloads.gaussian(workloads.rng(400 + seed, m), (m, k), 1.0)
    workloads.plant_scale_columns(x, workloads.rng(401 + seed, k), min(6, k), 50.0, 100.0)
    w = workloads.gaussian(workloads.rng(402 + seed, n), (n, k), 0.02)
    return workloads.to_dtype(x, xdt), workloads.to_dtype(w, wdt)


SMALL = [(1, 64, 1), (37, 192, 50), (130, 320, 129), (256, 1024, 300)]


@pytest.mark.parametrize("mkn", SMALL + [(2048, 4096, 4096)], ids=lambda t: "x".join(map(str, t)))
def test_smooth_factors(mkn):
    m, k, n = mkn
    x, w = sq_inputs(m, k, n)
    note(f"sq_smooth_factors M={m} K={k} N={n}")
    s, cx, cw = qmm.sq_smooth_factors(x.to(DEV), w.to(DEV), 0.5)
    rcx, rcw = oracle.col_absmax(x.float().numpy()), oracle.col_absmax(w.float().numpy())
    rs = oracle.smooth_factors(rcx, rcw, 0.5)
    assert bits_equal(cx.cpu().numpy(), rcx), first_diff(cx.cpu().numpy(), rcx)
    assert bits_equal(cw.cpu().numpy(), rcw), first_diff(cw.cpu().numpy(), rcw)
    assert bits_equal(s.cpu().numpy(), rs), first_diff(s.cpu().numpy(), rs)


def test_smooth_factors_other_alpha_and_dtypes():
    x, w = sq_inputs(64, 256, 96, "f32", "f16", seed=3)
    note("sq_smooth_factors alpha=0.75 f32/f16")
    s, cx, cw = qmm.sq_smooth_factors(x.to(DEV), w.to(DEV), 0.75)
    rs = oracle.smooth_factors(oracle.col_absmax(x.float().numpy()), oracle.col_absmax(w.float().numpy()), 0.75)
    # powf is not correctly rounded on either side: a few ulps
    assert np.allclose(s.cpu().numpy(), rs, rtol=4e-7 * 8, atol=0)


@pytest.mark.parametrize("smoothed", [True, False])
@pytest.mark.parametrize("mkn", SMALL + [(2048, 4096, 4096)], ids=lambda t: "x".join(map(str, t)))
def test_quantize_weight_and_activation(mkn, smoothed):
    m, k, n = mkn
    x, w = sq_inputs(m, k, n, seed=1)
    xf, wf = x.float().numpy(), w.float().numpy()
    rs = oracle.smooth_factors(oracle.col_absmax(xf), oracle.col_absmax(wf), 0.5) if smoothed else None
    sd = torch.from_numpy(rs).to(DEV) if smoothed else None
    note(f"sq_quantize_weight/activation M={m} K={k} N={n} smooth={smoothed}")
    qw, b = qmm.sq_quantize_weight(w.to(DEV), sd)
    qx, a = qmm.sq_quantize_activation(x.to(DEV), sd)
    rqw, rb = oracle.sq_quantize_weight(wf, rs)
    rqx, ra = oracle.sq_quantize_activation(xf, rs)
    assert bits_equal(b.cpu().numpy(), rb), first_diff(b.cpu().numpy(), rb)
    assert bits_equal(qw.cpu().numpy(), rqw), first_diff(qw.cpu().numpy(), rqw)
    assert bits_equal(a.cpu().numpy(), ra), first_diff(a.cpu().numpy(), ra)
    assert bits_equal(qx.cpu().numpy(), rqx), first_diff(qx.cpu().numpy(), rqx)


def test_quantize_activation_long_rows_and_zero_row():
    # rows longer than the register-resident path (second pass re-reads) and an all-zero row
    x = workloads.gaussian(workloads.rng(9, 9), (5, 8192), 1.0)
    x[2] = 0.0
    xb = workloads.to_dtype(x, "bf16")
    note("sq_quantize_activation 5x8192 with a zero row")
    qx, a = qmm.sq_quantize_activation(xb.to(DEV), None)
    rqx, ra = oracle.sq_quantize_activation(xb.float().numpy(), None)
    assert bits_equal(a.cpu().numpy(), ra) and bits_equal(qx.cpu().numpy(), rqx)


def test_quantize_activation_extreme_smoothing():
    # Activations divide by the smoothing factors through a reciprocal table:
    # factors outside [2^-100, 2^100] must take the exact division, quotients
    # far below 2^-102 (where the table form may differ in the last place)
    # must change no code and no scale, and a row under the 1e-8 absmax floor
    # keeps its floored scale.  fp32 input, so subnormals reach the kernel.
    k = 512
    g = np.random.Generator(np.random.PCG64(77))
    x = g.standard_normal((8, k)).astype(np.float32)
    sm = (g.random(k) + 0.5).astype(np.float32)
    sm[3], sm[17], sm[40], sm[41], sm[300] = 1e-33, 3e33, 2.0 ** -100, 2.0 ** 100, 2.0 ** -101
    x[1] *= np.float32(1e-36)            # quotients around 1e-36 and below
    x[2] *= np.float32(1e-40)            # subnormal inputs
    x[3] = np.float32(3e-9) * np.sign(x[3])   # absmax under the floor
    x[4] *= np.float32(1e4)              # quotients up to ~3e37 in the 1e-33 column
    x[5, ::3] = np.float32(1.5e-45)      # smallest subnormal among normal values
    note("sq_quantize_activation 8x512 fp32, extreme smoothing factors")
    qx, a = qmm.sq_quantize_activation(torch.from_numpy(x).to(DEV), torch.from_numpy(sm).to(DEV))
    rqx, ra = oracle.sq_quantize_activation(x, sm)
    assert bits_equal(a.cpu().numpy(), ra), first_diff(a.cpu().numpy(), ra)
    assert bits_equal(qx.cpu().numpy(), rqx), first_diff(qx.cpu().numpy(), rqx)


@pytest.mark.parametrize("mnk", [(1, 1, 64), (5, 7, 128), (130, 129, 320), (128, 128, 64), (300, 257, 1024),
                                 (64, 300, 384), (513, 130, 256), (257, 129, 448)],
                         ids=lambda t: "x".join(map(str, t)))
def test_int8_gemm_exact(mnk):
    m, n, k = mnk
    g = np.random.Generator(np.random.PCG64(m * 1000 + n))
    qa = g.integers(-128, 128, size=(m, k)).astype(np.int8)
    qb = g.integers(-128, 128, size=(n, k)).astype(np.int8)
    note(f"sq_int8_gemm int32 M={m} N={n} K={k}")
    acc = qmm.sq_int8_gemm(torch.from_numpy(qa).to(DEV), None, torch.from_numpy(qb).to(DEV), None,
                           out_dtype=torch.int32)
    ref = oracle.int8_matmul_nt(qa, qb)
    assert np.array_equal(acc.cpu().numpy(), ref), first_diff(acc.cpu().numpy(), ref)


def test_int8_gemm_extremes():
    # all -128 x -128 at the largest K the library accepts: the sums reach
    # 128 * 128 * K = 2146435072, just inside int32
    m, n, k = 16, 16, 131008
    qa = np.full((m, k), -128, np.int8)
    qb = np.full((n, k), -128, np.int8)
    qb[1] = 127
    note("sq_int8_gemm extremes K=131008")
    acc = qmm.sq_int8_gemm(torch.from_numpy(qa).to(DEV), None, torch.from_numpy(qb).to(DEV), None,
                           out_dtype=torch.int32).cpu().numpy()
    assert int(acc[0, 0]) == 128 * 128 * k == 2146435072
    assert int(acc[3, 1]) == -128 * 127 * k


@pytest.mark.parametrize("ydt", ["bf16", "f32"])
@pytest.mark.parametrize("mkn", SMALL + [(2048, 4096, 4096)], ids=lambda t: "x".join(map(str, t)))
def test_w8a8_pipeline(mkn, ydt):
    m, k, n = mkn
    x, w = sq_inputs(m, k, n, seed=2)
    xf, wf = x.float().numpy(), w.float().numpy()
    xd, wd = x.to(DEV), w.to(DEV)
    note(f"smooth_quant_w8a8_gemm M={m} K={k} N={n} y={ydt}")
    s, _, _ = qmm.sq_smooth_factors(xd, wd, 0.5)
    qw, b = qmm.sq_quantize_weight(wd, s)
    y = qmm.smooth_quant_w8a8_gemm(xd, s, qw, b, out_dtype=TDT[ydt])
    acc = qmm.sq_int8_gemm(*qmm.sq_quantize_activation(xd, s), qw, b, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rs = oracle.smooth_factors(oracle.col_absmax(xf), oracle.col_absmax(wf), 0.5)
    rqw, rb = oracle.sq_quantize_weight(wf, rs)
    # all tokens of the small cases; at 2048 tokens one row in every 32 (each
    # 256-row output tile sampled 8 times), all 4096 output columns
    rows = np.arange(m) if m <= 256 else stratified_rows(m, 32)
    rqx, ra = oracle.sq_quantize_activation(xf[rows], rs)
    racc = oracle.int8_matmul_nt(rqx, rqw)
    assert np.array_equal(acc.cpu().numpy()[rows], racc)
    ref = oracle.rescale_f64(racc, ra, rb)
    assert_close(y.cpu()[rows], ref, f"w8a8 {mkn} {ydt}")


def test_w8a8_no_smoothing_and_deterministic():
    x, w = sq_inputs(130, 320, 129, seed=4)
    xd, wd = x.to(DEV), w.to(DEV)
    note("smooth_quant_w8a8_gemm smooth=None")
    qw, b = qmm.sq_quantize_weight(wd, None)
    y1 = qmm.smooth_quant_w8a8_gemm(xd, None, qw, b, out_dtype=torch.float32).cpu()
    y2 = qmm.smooth_quant_w8a8_gemm(xd, None, qw, b, out_dtype=torch.float32).cpu()
    assert torch.equal(y1, y2)
    rqw, rb = oracle.sq_quantize_weight(w.float().numpy(), None)
    _, _, _, ref = oracle.sq_w8a8_reference(x.float().numpy(), None, rqw, rb)
    assert_close(y1, ref, "w8a8 no smoothing")


@pytest.mark.parametrize("smoothed", [True, False])
@pytest.mark.parametrize("mkn", SMALL + [(2048, 4096, 4096)], ids=lambda t: "x".join(map(str, t)))
def test_quantize_activation_per_tensor(mkn, smoothed):
    # one INT8 scale for the whole activation matrix, repeated per row
    m, k, n = mkn
    x, w = sq_inputs(m, k, n, seed=3)
    xf, wf = x.float().numpy(), w.float().numpy()
    rs = oracle.smooth_factors(oracle.col_absmax(xf), oracle.col_absmax(wf), 0.5) if smoothed else None
    sd = torch.from_numpy(rs).to(DEV) if smoothed else None
    note(f"sq_quantize_activation_per_tensor M={m} K={k} smooth={smoothed}")
    qx, a = qmm.sq_quantize_activation(x.to(DEV), sd, per_tensor=True)
    rqx, ra = oracle.sq_quantize_activation_per_tensor(xf, rs)
    assert bits_equal(a.cpu().numpy(), ra), first_diff(a.cpu().numpy(), ra)
    assert bits_equal(qx.cpu().numpy(), rqx), first_diff(qx.cpu().numpy(), rqx)


def test_w8a8_per_tensor_pipeline_and_fp32_rows():
    # per-tensor activations through the INT8 GEMM (consumed like per-token
    # scales), and fp32 input with rows longer than the register-resident path
    m, k, n = 300, 1024, 257
    x, w = sq_inputs(m, k, n, seed=4)
    xf, wf = x.float().numpy(), w.float().numpy()
    rs = oracle.smooth_factors(oracle.col_absmax(xf), oracle.col_absmax(wf), 0.5)
    sd = torch.from_numpy(rs).to(DEV)
    qw, b = qmm.sq_quantize_weight(w.to(DEV), sd)
    qx, a = qmm.sq_quantize_activation(x.to(DEV), sd, per_tensor=True)
    rqx, ra = oracle.sq_quantize_activation_per_tensor(xf, rs)
    rqw, rb = oracle.sq_quantize_weight(wf, rs)
    note("w8a8 per-tensor activations through sq_int8_gemm")
    y = qmm.sq_int8_gemm(qx, a, qw, b, out_dtype=torch.float32).cpu()
    ref = oracle.rescale_f64(oracle.int8_matmul_nt(rqx, rqw), ra, rb)
    from gpu_util import assert_close
    assert_close(y, ref, "w8a8 per-tensor")
    g = np.random.Generator(np.random.PCG64(8))
    xl = (g.standard_normal((9, 8192)) * 3).astype(np.float32)
    xl[4] = 0.0
    note("sq_quantize_activation_per_tensor 9x8192 fp32")
    qx2, a2 = qmm.sq_quantize_activation(torch.from_numpy(xl).to(DEV), None, per_tensor=True)
    rq2, ra2 = oracle.sq_quantize_activation_per_tensor(xl, None)
    assert bits_equal(a2.cpu().numpy(), ra2) and bits_equal(qx2.cpu().numpy(), rq2)
