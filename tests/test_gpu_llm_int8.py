"""GPU parity for LLM.int8() (vector-wise INT8 with the outlier feature
dimensions multiplied in 16-bit): the outlier list, the column factors and the
INT8 activations bit for bit against the CPU oracle, the product within the
elementwise tolerance, on small ragged shapes, the degenerate thresholds, a
cap below the number found, and the 2048 x 4096 x 4096 workload."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import assert_close, bits_equal, first_diff, note, stratified_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TAU = 6.0
_TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _acts(m, k, dtype, seed):
    """N(0, 1) activations with outlier features: whole columns scaled up (the
    systematic kind), one column large in a single token, one reaching the
    threshold exactly, one just below it."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = workloads.gaussian(g, (m, k), 1.0)
    x = np.clip(x, -5.5, 5.5)
    cols = g.choice(k, size=min(4, k), replace=False)
    x[:, cols[0]] *= np.float32(30.0)
    if k > 1:
        x[m // 2, cols[1]] = np.float32(-250.0)
    if k > 2:
        x[m - 1, cols[2]] = np.float32(TAU)
    if k > 3:
        x[0, cols[3]] = np.float32(5.9375)
    return workloads.to_dtype(x, dtype)


def _weights(n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    w = workloads.to_dtype(workloads.gaussian(g, (n, k), 0.02), "bf16").float().numpy()
    return oracle.sq_quantize_weight(w, None)


def _check_outliers(x, dtype, cap, what):
    xd = x.to(DEV)
    note(f"llm_int8_outliers {what} shape={tuple(x.shape)} {dtype} cap={cap}")
    factor, index, found = qmm.llm_int8_outliers(xd, TAU, cap)
    k = x.shape[1]
    qw0 = np.zeros((1, k), np.int8)
    ridx, rfound, rqx, ra, _ = oracle.llm_int8_reference(x.float().numpy(), qw0, np.ones(1, np.float32), TAU,
                                                         cap, dtype)
    assert found == rfound, (found, rfound)
    assert index.cpu().numpy().tolist() == ridx.tolist()
    want = np.ones(k, np.float32)
    want[ridx] = np.inf
    assert bits_equal(factor.cpu().numpy(), want), f"{what} factors: {first_diff(factor.cpu().numpy(), want)}"
    qx, a = qmm.sq_quantize_activation(xd, factor)
    torch.cuda.synchronize()
    assert bits_equal(a.cpu().numpy(), ra), f"{what} token scales: {first_diff(a.cpu().numpy(), ra)}"
    assert bits_equal(qx.cpu().numpy(), rqx), f"{what} X_q: {first_diff(qx.cpu().numpy(), rqx)}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 64), (77, 320), (300, 4160), (2, 8192)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_outliers_and_activation_codes(shape, dtype):
    x = _acts(shape[0], shape[1], dtype, 11 + shape[0])
    _check_outliers(x, dtype, None, "small")


def test_outliers_many_columns_and_cap():
    # more than one chunk of 1024 columns holding outliers (the rank carries
    # across chunks), then caps that cut the list inside and between chunks
    m, k = 33, 5120
    g = np.random.Generator(np.random.PCG64(5))
    x = np.clip(workloads.gaussian(g, (m, k), 1.0), -5.0, 5.0)
    cols = np.sort(g.choice(k, size=300, replace=False))
    x[g.integers(0, m, size=cols.size), cols] = np.float32(40.0)
    xt = workloads.to_dtype(x, "bf16")
    for cap in (None, 299, 137, 1, 0):
        _check_outliers(xt, "bf16", cap, f"cap {cap}")


def _gemm_case(x, dtype, qw, b, cap, out, what, tau=TAU):
    M, K = x.shape
    N = qw.shape[0]
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    note(f"llm_int8_gemm {what} {M}x{N}x{K} {dtype} out={out} cap={cap} tau={tau}")
    y = qmm.llm_int8_gemm(x.to(DEV), torch.from_numpy(qw).to(DEV), torch.from_numpy(b).to(DEV), tau, cap,
                          out_dtype=odt, n_outliers=nt)
    torch.cuda.synchronize()
    ridx, rfound, _, _, ry = oracle.llm_int8_reference(x.float().numpy(), qw, b, tau, cap, dtype)
    assert int(nt.item()) == rfound
    assert_close(y, ry, f"llm_int8 {what} {M}x{N}x{K} {out}")
    return y, ridx


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mnk", [(1, 64, 64), (16, 300, 320), (77, 520, 1024), (300, 257, 4160)],
                         ids=lambda t: "x".join(map(str, t)))
def test_llm_int8_gemm_small(mnk, dtype, out):
    M, N, K = mnk
    x = _acts(M, K, dtype, 20 + M)
    qw, b = _weights(N, K, 30 + N)
    _gemm_case(x, dtype, qw, b, None, out, "small")


def test_llm_int8_degenerate_thresholds():
    M, N, K = 77, 130, 640
    x = _acts(M, K, "bf16", 3)
    qw, b = _weights(N, K, 4)
    # no outlier dimension: the plain vector-wise W8A8 product, bit for bit
    y, ridx = _gemm_case(x, "bf16", qw, b, None, "f32", "threshold inf", tau=float("inf"))
    assert len(ridx) == 0
    y0 = qmm.smooth_quant_w8a8_gemm(x.to(DEV), None, torch.from_numpy(qw).to(DEV), torch.from_numpy(b).to(DEV),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    # every column an outlier: the whole product in 16-bit, the integer part empty
    for dtype in ("bf16", "f16"):
        xd = _acts(M, K, dtype, 5)
        _, ridx = _gemm_case(xd, dtype, qw, b, None, "f32", "threshold 0", tau=0.0)
        assert len(ridx) == K


def test_llm_int8_cap_and_workspace_reuse():
    # a cap below the number found, then a second, smaller call through the
    # same workspace (nothing in it needs clearing between calls)
    M, N, K = 150, 200, 1088
    qw, b = _weights(N, K, 6)
    x1 = _acts(M, K, "bf16", 7)
    g = np.random.Generator(np.random.PCG64(8))
    x1n = x1.float().numpy()
    x1n[3, g.choice(K, size=20, replace=False)] = 80.0
    x1 = workloads.to_dtype(x1n, "bf16")
    ws = torch.empty(qmm.llm_int8_workspace_bytes(M, N, K, 8), dtype=torch.uint8, device=DEV)
    dq, db = torch.from_numpy(qw).to(DEV), torch.from_numpy(b).to(DEV)
    for xx, m, cap in ((x1, M, 8), (_acts(40, K, "bf16", 9), 40, 3)):
        note(f"llm_int8_gemm workspace reuse M={m} cap={cap}")
        y = qmm.llm_int8_gemm(xx.to(DEV), dq, db, TAU, cap, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        ridx, rfound, _, _, ry = oracle.llm_int8_reference(xx.float().numpy(), qw, b, TAU, cap, "bf16")
        assert len(ridx) == min(cap, rfound)
        assert_close(y, ry, f"llm_int8 reuse M={m} cap={cap}")


def test_llm_int8_full_size():
    # the W8A8 workload's shapes (2048 x 4096 x 4096, six outlier channels x
    # 50..100): the outlier list is exactly the planted channels, X_q and the
    # token scales bit for bit, the product on rows meeting every 256-row tile
    wl = workloads.WORKLOADS["smoothquant"]
    M, N, K = 2048, 4096, 4096
    x, cols = workloads.sq_activations(wl, M, K)
    w, _ = workloads.weight(wl, 0)
    qw, b = oracle.sq_quantize_weight(w.float().numpy(), None)
    xn = x.float().numpy()
    want = np.nonzero(oracle.col_absmax(xn) >= TAU)[0]
    assert want.tolist() == sorted(int(c) for c in cols)
    _check_outliers(x, "bf16", None, "full")
    note("llm_int8_gemm 2048x4096x4096")
    xd, dq, db = x.to(DEV), torch.from_numpy(qw).to(DEV), torch.from_numpy(b).to(DEV)
    nt = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = qmm.llm_int8_gemm(xd, dq, db, TAU, out_dtype=torch.float32, n_outliers=nt)
    yb = qmm.llm_int8_gemm(xd, dq, db, TAU)
    torch.cuda.synchronize()
    assert int(nt.item()) == 6
    rows = stratified_rows(M, 32)
    ridx, _, _, _, ry = oracle.llm_int8_reference(xn[rows], qw, b, TAU)
    assert ridx.tolist() == want.tolist()      # the sample sees the batch's outlier set
    sel = torch.from_numpy(rows)
    assert_close(y.cpu()[sel], ry, "llm_int8 full size f32")
    assert_close(yb.cpu()[sel], ry, "llm_int8 full size bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_llm_int8_outliers_past_the_staged_ones(dtype):
    # 23 outlier columns: the GEMM stages the first ones beside its LDS tiles
    # and reads the rest straight from X and the weights; ragged M and N
    M, N, K = 300, 390, 1152
    g = np.random.Generator(np.random.PCG64(31))
    x = np.clip(workloads.gaussian(g, (M, K), 1.0), -5.0, 5.0)
    cols = np.sort(g.choice(K, size=23, replace=False))
    x[g.integers(0, M, size=cols.size), cols] = np.float32(-60.0)
    qw, b = _weights(N, K, 32)
    _, ridx = _gemm_case(workloads.to_dtype(x, dtype), dtype, qw, b, None, "f32", "23 outliers")
    assert len(ridx) == 23
