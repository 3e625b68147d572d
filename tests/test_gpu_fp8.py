"""GPU parity for FP8 E4M3 W8A8: quantizer codes and scales bit for bit
against the CPU oracle (per row and per tensor), the FP8 GEMM and the online
call within the elementwise tolerance."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import assert_close, bits_equal, first_diff, note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
# The fp8 matrix instruction sums its products with fewer bits than an fp32
# accumulation (measured: norm-wise relative error ~5e-5 against the exact
# product even at K = 64, where fp32 rounding alone gives ~1e-7), so the
# norm-wise check of fp32 outputs uses 2e-4; the elementwise bound (1e-3 of
# the value plus 1e-3 of the rms) is the one every matmul meets.
FP8_NORMWISE = 2e-4


def _compare_quant(x_cpu, per_tensor, what):
    note(f"fp8_quantize {what} shape={tuple(x_cpu.shape)} {x_cpu.dtype} per_tensor={per_tensor}")
    q, s = qmm.fp8_quantize(x_cpu.to(DEV), per_tensor)
    torch.cuda.synchronize()
    rq, rs = oracle.fp8_quantize(x_cpu.float().numpy(), per_tensor)
    assert bits_equal(s.cpu().numpy(), rs), f"{what} scales: {first_diff(s.cpu().numpy(), rs)}"
    assert bits_equal(q.cpu().numpy(), rq), f"{what} codes: {first_diff(q.cpu().numpy(), rq)}"
    return q, s, rq, rs


@pytest.mark.parametrize("per_tensor", [False, True], ids=["per_row", "per_tensor"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(1, 64), (77, 320), (300, 4160), (5, 8192)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fp8_quantize_small(shape, dtype, per_tensor):
    g = workloads.rng(88, shape[0] + shape[1])
    x = workloads.gaussian(g, shape, 1.0)
    x[:, :: max(1, shape[1] // 7)] *= np.float32(60.0)        # outlier channels
    _compare_quant(workloads.to_dtype(x, dtype), per_tensor, f"small-{dtype}")


def test_fp8_quantize_edges():
    # an all-zero row (absmax floor), a row whose quotients reach E4M3's
    # subnormals and exact ties, a row of one huge and many tiny values, and
    # the values at 448's neighbourhood
    k = 512
    x = np.zeros((6, k), np.float32)
    x[1] = np.linspace(-1.0, 1.0, k) * np.float32(2.0 ** -12)
    x[1, 0] = 1.0
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.from_e4m3(codes)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    x[2, :len(mids)] = mids
    x[2, -1] = 448.0                                           # scale exactly 1: the ties stay ties
    x[3, 0] = 1e4
    x[3, 1:] = np.float32(1e-3)
    x[4] = np.float32(447.99) * np.sign(np.linspace(-1, 1, k) + 1e-3)
    x[5] = np.random.Generator(np.random.PCG64(4)).standard_normal(k).astype(np.float32) * np.float32(1e-30)
    for per_tensor in (False, True):
        _compare_quant(torch.from_numpy(x), per_tensor, "edges")


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("mnk", [(16, 64, 64), (77, 300, 320), (256, 128, 1024), (300, 520, 4160)],
                         ids=lambda t: "x".join(map(str, t)))
def test_fp8_gemm_small(mnk, out):
    M, N, K = mnk
    wl = workloads.WORKLOADS["smoothquant"]
    x, _ = workloads.sq_activations(wl, M, K)
    w, _ = workloads.weight(wl, 0, shape=(N, K))
    qx, sx, rqx, rsx = _compare_quant(x, False, "gemm-x")
    qw, sw, rqw, rsw = _compare_quant(w, False, "gemm-w")
    note(f"fp8_gemm {M}x{N}x{K} out={out}")
    y = qmm.fp8_gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = oracle.fp8_matmul_nt(rqx, rqw) * rsx.astype(np.float64)[:, None] * rsw.astype(np.float64)[None, :]
    assert_close(y, ref, f"fp8_gemm {mnk} {out}", normwise=FP8_NORMWISE)


def test_fp8_gemm_exact_products():
    # codes whose values are small integers: every product and (fp32) partial
    # sum is exact, so the raw product (unit scales, fp32 out) equals the
    # oracle's exactly
    g = np.random.Generator(np.random.PCG64(12))
    vals = np.float32([0, 1, -1, 2, -2, 3, -4, 0.5])
    M, N, K = 96, 200, 640
    a = vals[g.integers(0, len(vals), (M, K))]
    b = vals[g.integers(0, len(vals), (N, K))]
    qa, qb = oracle.to_e4m3(a), oracle.to_e4m3(b)
    note("fp8_gemm exact small-integer products")
    y = qmm.fp8_gemm(torch.from_numpy(qa).to(DEV), torch.ones(M, device=DEV), torch.from_numpy(qb).to(DEV),
                     torch.ones(N, device=DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.fp8_matmul_nt(qa, qb))


def test_fp8_w8a8_full_size():
    # the SmoothQuant workload's shapes (2048 x 4096 x 4096, activations with
    # outlier channels), weights per output channel, activations per token;
    # codes and scales bit for bit, outputs on 64 rows covering every
    # 256-row output tile
    wl = workloads.WORKLOADS["smoothquant"]
    M, N, K = 2048, 4096, 4096
    x, _ = workloads.sq_activations(wl, M, K)
    w, _ = workloads.weight(wl, 0)
    qw, sw, rqw, rsw = _compare_quant(w, False, "full-w")
    _compare_quant(x, False, "full-x")
    note("fp8_w8a8_gemm 2048x4096x4096")
    xd = x.to(DEV)
    y = qmm.fp8_w8a8_gemm(xd, qw, sw, out_dtype=torch.float32)
    yb = qmm.fp8_w8a8_gemm(xd, qw, sw)
    torch.cuda.synchronize()
    rows = np.arange(0, M, 32) + (np.arange(M // 32) % 32)
    _, _, ref = oracle.fp8_w8a8_reference(x.float().numpy()[rows], rqw, rsw)
    assert_close(y.cpu()[torch.from_numpy(rows)], ref, "fp8_w8a8 full size f32", normwise=FP8_NORMWISE)
    assert_close(yb.cpu()[torch.from_numpy(rows)], ref, "fp8_w8a8 full size bf16")


def test_fp8_argument_errors():
    lib = qmm.lib()
    P = qmm._ptr(torch.empty(64, dtype=torch.uint8, device=DEV))
    assert lib.fp8_gemm(P, P, P, P, 4, 4, 100, P, qmm.BF16, None) == -2          # K % 64
    assert lib.fp8_gemm(P, P, P, P, 4, 4, 64, P, qmm.I32, None) == -2            # no raw int output
    assert lib.fp8_gemm(P, None, P, P, 4, 4, 64, P, qmm.BF16, None) == -1        # scales required
    assert lib.fp8_w8a8_gemm(P, qmm.BF16, P, P, 4, 4, 64, P, qmm.BF16, P, 16, None) == -4   # workspace


def test_fp8_gemm_tail_keeps_rows_apart():
    # K % 128 == 64: the second half of the last k-step lies past the end of
    # every row (the next row's first bytes).  NaN codes at the start of one
    # row of each operand must reach only that row's outputs; every other
    # output equals the exact product.
    g = np.random.Generator(np.random.PCG64(14))
    M, N, K = 40, 72, 192
    vals = np.float32([0, 1, -1, 2, -2, 0.5, 4])
    a = vals[g.integers(0, len(vals), (M, K))]
    b = vals[g.integers(0, len(vals), (N, K))]
    qa, qb = oracle.to_e4m3(a), oracle.to_e4m3(b)
    qa[7, 0] = 0x7F                                   # E4M3FN NaN
    qb[11, 3] = 0xFF
    note("fp8_gemm NaN codes next to the K tail")
    y = qmm.fp8_gemm(torch.from_numpy(qa).to(DEV), torch.ones(M, device=DEV), torch.from_numpy(qb).to(DEV),
                     torch.ones(N, device=DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.fp8_matmul_nt(qa, qb)
    yv = y.cpu().numpy().astype(np.float64)
    poisoned = np.zeros((M, N), bool)
    poisoned[7, :] = True
    poisoned[:, 11] = True
    assert np.isnan(ref[poisoned]).all() and np.isnan(yv[poisoned]).all()
    assert np.array_equal(yv[~poisoned], ref[~poisoned])
