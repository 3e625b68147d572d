"""W8A16 weight-only INT8 GEMV against the oracle (fp64 sums; tolerance as for
the INT4 matmuls: 1e-3 relative with fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import stratified_rows, assert_close, bits_equal, first_diff, note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def random_w8(n, k, seed):
    g = workloads.rng(90, seed)
    q = g.integers(-128, 128, (n, k)).astype(np.int8)
    b = (g.random(n) * 0.02 + 1e-3).astype(np.float32)
    return q, b


def w8_case(q, b, x_cpu, ydt, what, rows=None):
    note(f"w8a16_gemv {what} N={q.shape[0]} K={q.shape[1]} B={x_cpu.shape[0]} x={x_cpu.dtype} y={ydt}")
    y = qmm.w8a16_gemv(torch.from_numpy(q).to(DEV), torch.from_numpy(b).to(DEV), x_cpu.to(DEV), out_dtype=ydt)
    torch.cuda.synchronize()
    xf = x_cpu.float().numpy()
    if rows is None:
        return assert_close(y.cpu(), oracle.w8a16_reference(xf, q, b), what)
    return assert_close(y.cpu()[:, rows], oracle.w8a16_reference(xf, q[rows], b[rows]), what)


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("ysame", [True, False], ids=["y=x", "y=f32"])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("shape", [(1, 64), (7, 192), (37, 4160), (130, 8256), (9, 12352)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_w8a16_small(xdt, ysame, B, shape):
    # rows around the 8-row block, K from one 64-wide slice to three 4096-wide
    # steps plus a ragged tail (lanes past K, wavefronts with nothing to do)
    n, k = shape
    q, b = random_w8(n, k, seed=n * 7 + k + B)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(91, n + k + B), (B, k), 1.0), xdt)
    w8_case(q, b, x, TDT[xdt] if ysame else torch.float32, f"small {xdt}")


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("ysame", [True, False], ids=["y=x", "y=f32"])
@pytest.mark.parametrize("B", [3, 5, 8])
@pytest.mark.parametrize("shape", [(1, 256), (37, 768), (130, 1280), (16, 4352), (45, 8448)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_w8a16_staged(xdt, ysame, B, shape):
    # K a multiple of 256 (the LDS-staged matrix-core kernel): one step (three
    # wavefronts idle), three and five steps over four wavefronts (one or two
    # idle or short), 17 and 33 steps; rows ragged around the 16-row block
    n, k = shape
    q, b = random_w8(n, k, seed=n * 11 + k + B)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(96, n + k + B), (B, k), 1.0), xdt)
    w8_case(q, b, x, TDT[xdt] if ysame else torch.float32, f"staged {xdt}")


def test_w8a16_extreme_codes():
    # every weight at -128 or 127 and large activations: the fp32 sums of the
    # exact products stay within the bound
    n, k = 24, 8192
    q = np.where(workloads.rng(92, 0).random((n, k)) < 0.5, -128, 127).astype(np.int8)
    b = np.full(n, 0.25, np.float32)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(93, 0), (8, k), 100.0), "bf16")
    w8_case(q, b, x[:1], torch.float32, "extreme B=1")
    w8_case(q, b, x, torch.float32, "extreme B=8")


def test_w8a16_after_weight_quantizer():
    # the on-device per-channel quantizer (no smoothing) feeds the GEMV; its
    # codes and scales match the oracle bit for bit
    n, k = 300, 4096
    w = workloads.to_dtype(workloads.gaussian(workloads.rng(94, 0), (n, k), 0.02), "bf16")
    qd, bd = qmm.sq_quantize_weight(w.to(DEV))
    qo, bo = oracle.sq_quantize_weight(w.float().numpy(), None)
    assert bits_equal(qd.cpu().numpy(), qo), first_diff(qd.cpu().numpy(), qo)
    assert bits_equal(bd.cpu().numpy(), bo), first_diff(bd.cpu().numpy(), bo)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(95, 0), (4, k), 1.0), "bf16")
    y = qmm.w8a16_gemv(qd, bd, x.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y.cpu(), oracle.w8a16_reference(x.float().numpy(), qo, bo), "after quantizer")


@pytest.mark.parametrize("index,B", [(0, 1), (1, 1), (0, 8), (1, 8)])
def test_w8a16_full_size(index, B):
    # the 70B-class MLP matrices at full size: quantized on the device, codes
    # and outputs checked on one row of every 8-row block
    wl = workloads.WORKLOADS["mlp70b"]
    w, _ = workloads.weight(wl, index)
    n, k = w.shape
    note(f"w8a16 full size mlp70b[{index}] {n}x{k} B={B}")
    wd = w.to(DEV)
    qd, bd = qmm.sq_quantize_weight(wd)
    del wd
    rows = stratified_rows(n, 8)          # one row in every 8-row block of the kernels
    qo, bo = oracle.sq_quantize_weight(w[rows].float().numpy(), None)
    qs = qd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert bits_equal(qs, qo), first_diff(qs, qo)
    assert bits_equal(bd.cpu().numpy()[rows], bo)
    x = workloads.activations(wl, B, k, salt=index)
    ydt = torch.float16 if wl.x_dtype == "f16" else torch.bfloat16
    for out in (torch.float32, ydt):
        y = qmm.w8a16_gemv(qd, bd, x.to(DEV), out_dtype=out)
        torch.cuda.synchronize()
        assert_close(y.cpu()[:, rows], oracle.w8a16_reference(x.float().numpy(), qo, bo), f"full {index} B={B} {out}")
