"""smooth_quant_w8a8_gemm_noalloc (library-owned device scratch) against
smooth_quant_w8a8_gemm (caller workspace), called through the C ABI.

Both run the same kernels on the same operands, so the outputs must agree
bit for bit; the first call is the full SmoothQuant workload (2048 x 4096 x
4096, 8 MiB of quantized activations in the scratch), the second a smaller
ragged one, so the second call runs on scratch that still holds the first
call's bytes.  A size beyond the scratch is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import bits_equal, first_diff, note

pytestmark = pytest.mark.gpu

ERANGE = -6


def _operands(M, N, K, dev):
    wl = workloads.WORKLOADS["smoothquant"]
    x, _ = workloads.sq_activations(wl, M, K)
    w, _ = workloads.weight(wl, 0, shape=(N, K))
    x, w = x.to(dev), w.to(dev)
    smooth, _, _ = qmm.sq_smooth_factors(x, w)
    qw, wsc = qmm.sq_quantize_weight(w, smooth)
    return x, smooth, qw, wsc


def _both(x, smooth, qw, wsc, y_dtype):
    lib = qmm.lib()
    M, K = x.shape
    N = qw.shape[0]
    dt = qmm._dt(y_dtype)
    ws = torch.empty(qmm.sq_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
    y_ref = torch.full((M, N), 7, dtype=y_dtype, device=x.device)
    y = torch.full((M, N), 3, dtype=y_dtype, device=x.device)
    st = lib.smooth_quant_w8a8_gemm(qmm._ptr(x), qmm.BF16, qmm._ptr(smooth), qmm._ptr(qw), qmm._ptr(wsc), M, N, K,
                                    qmm._ptr(y_ref), dt, qmm._ptr(ws), ws.numel(), qmm._stream(x))
    assert st == 0, st
    st = lib.smooth_quant_w8a8_gemm_noalloc(qmm._ptr(x), qmm.BF16, qmm._ptr(smooth), qmm._ptr(qw), qmm._ptr(wsc),
                                            M, N, K, qmm._ptr(y), dt, qmm._stream(x))
    assert st == 0, st
    torch.cuda.synchronize()
    return y.cpu(), y_ref.cpu()


@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.int32], ids=["bf16", "i32"])
def test_noalloc_matches_workspace_call(y_dtype):
    dev = torch.device("cuda:0")
    for M, N, K in [(2048, 4096, 4096), (77, 320, 1152)]:
        note(f"w8a8 noalloc vs workspace: M={M} N={N} K={K} out={y_dtype}")
        x, smooth, qw, wsc = _operands(M, N, K, dev)
        y, y_ref = _both(x, smooth, qw, wsc, y_dtype)
        a, b = y.view(torch.int16 if y.element_size() == 2 else torch.int32).numpy(), \
            y_ref.view(torch.int16 if y.element_size() == 2 else torch.int32).numpy()
        assert bits_equal(a, b), first_diff(a, b)


def test_noalloc_refuses_sizes_beyond_scratch():
    dev = torch.device("cuda:0")
    lib = qmm.lib()
    M, N, K = 4160, 64, 4096          # M*K = 17 039 360 > the scratch
    assert qmm.sq_workspace_bytes(M, K) > qmm.SQ_STATIC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    qw = torch.zeros((N, K), dtype=torch.int8, device=dev)
    wsc = torch.ones(N, dtype=torch.float32, device=dev)
    y = torch.full((M, N), 5, dtype=torch.bfloat16, device=dev)
    note("w8a8 noalloc: size beyond the scratch is refused")
    st = lib.smooth_quant_w8a8_gemm_noalloc(qmm._ptr(x), qmm.BF16, None, qmm._ptr(qw), qmm._ptr(wsc), M, N, K,
                                            qmm._ptr(y), qmm.BF16, qmm._stream(x))
    assert st == ERANGE
    torch.cuda.synchronize()
    assert (y == 5).all()               # nothing was written
    # the largest M at this K that fits still runs
    M2 = 4096
    assert qmm.sq_workspace_bytes(M2, K) <= qmm.SQ_STATIC_SCRATCH_BYTES
    x2, smooth2, qw2, wsc2 = _operands(M2, 128, K, dev)
    y2, y2_ref = _both(x2, smooth2, qw2, wsc2, torch.bfloat16)
    assert bits_equal(y2.view(torch.int16).numpy(), y2_ref.view(torch.int16).numpy())
