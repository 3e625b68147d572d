"""GPU parity: W4A16 GEMV / GEMM against the oracle's fp64 product with the dequantized weights."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import assert_close, note, random_w4, stratified_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def upload_w4(q, s, z):
    return (torch.from_numpy(oracle.pack_codes(q)).to(DEV), torch.from_numpy(np.ascontiguousarray(s)).to(DEV),
            torch.from_numpy(oracle.pack_nibbles(z)).to(DEV))


def gemv_case(q, s, z, x_cpu, ydt, what, gemm=False, rows=None):
    codes, scales, zeros = upload_w4(q, s, z)
    note(f"{'w4a16_gemm' if gemm else 'w4a16_gemv'} {what} N={q.shape[0]} K={q.shape[1]} "
         f"B={x_cpu.shape[0]} x={x_cpu.dtype} y={ydt}")
    xd = x_cpu.to(DEV)
    fn = qmm.w4a16_gemm if gemm else qmm.w4a16_gemv
    y = fn(codes, scales, zeros, xd, out_dtype=ydt)
    torch.cuda.synchronize()
    xf = x_cpu.float().numpy()
    if rows is None:
        ref = oracle.w4a16_reference(xf, q, s, z)
        return assert_close(y.cpu(), ref, what)
    ref = oracle.w4a16_reference(xf, q[rows], s[rows], z[rows])
    return assert_close(y.cpu()[:, rows], ref, what)


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("ysame", [True, False], ids=["y=x", "y=f32"])
@pytest.mark.parametrize("B", [1, 2, 3, 8])
@pytest.mark.parametrize("shape", workloads.shapes_for_parity(), ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemv_small(xdt, ysame, B, shape):
    n, k = shape
    q, s, z = random_w4(n, k, seed=n * 31 + k + B)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(77, n + B), (B, k), 1.0), xdt)
    gemv_case(q, s, z, x, TDT[xdt] if ysame else torch.float32, f"small {xdt}")


@pytest.mark.parametrize("k", [8320, 12672, 18560, 28672])
def test_gemv_long_k(k):
    # K beyond one 8192-wide step: the single-token kernel pipelines its steps,
    # with partly covered and skipped last steps per wavefront
    n = 37
    q, s, z = random_w4(n, k, seed=k)
    for xdt in ("bf16", "f16"):
        x = workloads.to_dtype(workloads.gaussian(workloads.rng(80, k), (1, k), 1.0), xdt)
        gemv_case(q, s, z, x, torch.float32, f"long K {xdt}")
        gemv_case(q, s, z, x, TDT[xdt], f"long K {xdt} 16-bit")


@pytest.mark.parametrize("k", [128, 1152, 2048, 2176, 4096, 6144, 6272])
@pytest.mark.parametrize("B", [1, 2])
def test_gemv_k_split_boundaries(k, B):
    # The single-token kernel splits K over one, two or four wavefronts by K
    # (at most 2048, at most 6144, above); the other wavefronts of a block take
    # more rows.  Row counts not a multiple of a block's rows leave sets empty.
    for n in (5, 45, 77):
        q, s, z = random_w4(n, k, seed=n * 7 + k + B)
        for xdt in ("bf16", "f16"):
            x = workloads.to_dtype(workloads.gaussian(workloads.rng(81, k + n), (B, k), 1.0), xdt)
            gemv_case(q, s, z, x, torch.float32, f"K split {xdt}")
            gemv_case(q, s, z, x, TDT[xdt], f"K split {xdt} 16-bit")


def test_gemv_one_row_one_group():
    q, s, z = random_w4(1, 128, seed=1)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(1, 1), (1, 128), 1.0), "bf16")
    gemv_case(q, s, z, x, torch.float32, "1x128")


def test_gemv_extreme_codes():
    # every code and zero-point at the ends of the range, large activations
    n, k = 40, 1024
    q = np.where(np.arange(n * k).reshape(n, k) % 3 == 0, 15, 0).astype(np.uint8)
    z = np.tile(np.array([0, 15], np.uint8), (n, k // 256))
    s = np.full((n, k // 128), 0.5, np.float32)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(3, 3), (8, k), 100.0), "bf16")
    gemv_case(q, s, z, x[:1], torch.float32, "extreme B=1")
    gemv_case(q, s, z, x, torch.float32, "extreme B=8")


def quantized(wl, index):
    w, _ = workloads.weight(wl, index)
    q, s, z = oracle.asym_quantize(w.float().numpy())
    return q, s, z


@pytest.mark.parametrize("name,index,B", [("tiny", 0, 1), ("llama7b", 0, 1), ("llama7b", 1, 1),
                                          ("mlp70b", 0, 1), ("mlp70b", 1, 1), ("mlp70b", 0, 2), ("mlp70b", 1, 2),
                                          ("mlp70b", 0, 8), ("mlp70b", 1, 8)])
def test_gemv_full_size(name, index, B):
    wl = workloads.WORKLOADS[name]
    q, s, z = quantized(wl, index)
    n, k = q.shape
    x = workloads.activations(wl, B, k, salt=index)
    # B = 1: every row; more tokens: one row in every block of 8 (the row
    # blocks of the vector-ALU kernel; each 16- or 32-row tile of the MFMA kernels)
    rows = None if B == 1 else stratified_rows(n, 8)
    ydt = torch.float16 if wl.x_dtype == "f16" else torch.bfloat16
    gemv_case(q, s, z, x, torch.float32, f"{name}[{index}] B={B} f32", rows=rows)
    gemv_case(q, s, z, x, ydt, f"{name}[{index}] B={B} 16-bit", rows=rows)


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 64, 100, 256])
@pytest.mark.parametrize("shape", [(3, 384), (129, 2176), (300, 1024), (64, 128), (65, 640)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemm_small(xdt, M, shape):
    # weight rows around the 64-row block tile, K from one group (fewer groups
    # than the block's four wavefronts) to 17 groups (uneven split)
    n, k = shape
    q, s, z = random_w4(n, k, seed=M * 13 + n)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(78, M + n), (M, k), 1.0), xdt)
    gemv_case(q, s, z, x, torch.float32, f"gemm small M={M}", gemm=True)
    gemv_case(q, s, z, x, TDT[xdt], f"gemm small M={M} {xdt}", gemm=True)


@pytest.mark.parametrize("M", [5, 40, 100, 200])
def test_gemm_wide_ragged(M):
    # enough weight rows that the split-K kernel takes 64 rows per block (the
    # small shapes above get 32-row blocks) and, for M = 100 and 200, that the
    # shared-tile kernel runs (64 x 128 tiles, ragged in M); a 37-row tail
    n, k = 257 * 64 + 37 - 64, 384
    q, s, z = random_w4(n, k, seed=M + 3)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(79, M), (M, k), 1.0), "bf16")
    gemv_case(q, s, z, x, torch.float32, f"gemm wide M={M}", gemm=True)
    gemv_case(q, s, z, x, torch.bfloat16, f"gemm wide M={M} bf16", gemm=True)


@pytest.mark.parametrize("M,n,k,xdt", [(2048, 4096, 4096, "bf16"), (1100, 6600, 1152, "f16"), (512, 33000, 640, "bf16")],
                         ids=["M2048-4096x4096", "M1100-6600x1152-f16", "M512-33000x640"])
def test_gemm_large_batch(M, n, k, xdt):
    # prefill-sized batches (the shared-tile kernel with many token tiles):
    # ragged M and N, an odd number of groups, both activation types; the
    # 4096-row case on rows that meet every 128-row tile
    q, s, z = random_w4(n, k, seed=M + n)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(83, M + k), (M, k), 1.0), xdt)
    rows = stratified_rows(n, 128) if M * n * k > 10 ** 10 else None
    gemv_case(q, s, z, x, torch.float32, f"gemm large M={M}", gemm=True, rows=rows)
    gemv_case(q, s, z, x, TDT[xdt], f"gemm large M={M} {xdt}", gemm=True, rows=rows)


@pytest.mark.parametrize("n", [12321, 16421], ids=["one block per CU", "two rounds of blocks"])
@pytest.mark.parametrize("M,k", [(3, 640), (16, 640), (17, 640), (32, 640), (40, 640), (64, 640), (16, 1152),
                                 (30, 1152), (50, 1152)], ids=lambda v: str(v))
def test_gemm_few_tokens_cooperative(n, M, k):
    # enough weight rows for the cooperative-load kernel (up to 64 tokens in
    # 16-, 32- or 64-token tiles; two or four groups per step): K = 5 or 9
    # groups, so the last step is partly past K; ragged N and M
    q, s, z = random_w4(n, k, seed=n + M)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(81, n + M), (M, k), 1.0), "bf16")
    gemv_case(q, s, z, x, torch.float32, f"gemm few tokens n={n} M={M}", gemm=True)
    gemv_case(q, s, z, x, torch.bfloat16, f"gemm few tokens n={n} M={M} bf16", gemm=True)


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("M,k", [(20, 53376), (7, 384128)], ids=["M20-K53376", "M7-K384128"])
def test_gemm_long_k_fallback(xdt, M, k):
    # K past what the LDS zero-point table of the tiled kernels holds (52224
    # for more than 16 tokens, 384000 for up to 16): the table-free kernel
    # serves both activation types; 37 rows, ragged against its row tiles
    n = 37
    q, s, z = random_w4(n, k, seed=k + M)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(82, k + M), (M, k), 1.0), xdt)
    gemv_case(q, s, z, x, torch.float32, f"gemm long K {xdt}", gemm=True)
    gemv_case(q, s, z, x, TDT[xdt], f"gemm long K {xdt} 16-bit", gemm=True)


@pytest.mark.parametrize("M", [16, 64, 256])
def test_gemm_full_size(M):
    # M = 16 and 64: every output; M = 256: one weight row in every 16 (each
    # 128-row tile of the shared-tile kernel sampled 8 times, at every row
    # position within a 16-row MFMA slice), all 256 tokens
    wl = workloads.WORKLOADS["gemm"]
    q, s, z = quantized(wl, 0)
    n, k = q.shape
    x = workloads.activations(wl, M, k)
    rows = None if M <= 64 else stratified_rows(n, 16)
    codes, scales, zeros = upload_w4(q, s, z)
    xd = x.to(DEV)
    ref = oracle.w4a16_reference(x.float().numpy(), *(a if rows is None else a[rows] for a in (q, s, z)))
    for ydt in (torch.bfloat16, torch.float32):
        note(f"w4a16_gemm 14336x4096 M={M} y={ydt} ({'all rows' if rows is None else f'{len(rows)} rows'})")
        y = qmm.w4a16_gemm(codes, scales, zeros, xd, out_dtype=ydt).cpu()
        assert_close(y if rows is None else y[:, rows], ref, f"gemm 14336x4096 M={M} {ydt}")


def test_gemm_m1_equals_gemv():
    wl = workloads.WORKLOADS["llama7b"]
    q, s, z = random_w4(257, 4224, seed=4)
    codes, scales, zeros = upload_w4(q, s, z)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(5, 5), (1, 4224), 1.0), "bf16").to(DEV)
    note("gemm M=1 vs gemv")
    a = qmm.w4a16_gemv(codes, scales, zeros, x, out_dtype=torch.float32).cpu().numpy()
    b = qmm.w4a16_gemm(codes, scales, zeros, x, out_dtype=torch.float32).cpu().numpy()
    assert np.allclose(a, b, rtol=1e-5, atol=1e-5 * np.abs(a).max())


def test_gemv_gemm_deterministic():
    q, s, z = random_w4(4096, 4096, seed=9)
    codes, scales, zeros = upload_w4(q, s, z)
    x = workloads.to_dtype(workloads.gaussian(workloads.rng(6, 6), (64, 4096), 1.0), "bf16").to(DEV)
    note("determinism gemv/gemm 4096x4096")
    for fn, xx in [(qmm.w4a16_gemv, x[:1]), (qmm.w4a16_gemv, x[:8]), (qmm.w4a16_gemm, x)]:
        a = fn(codes, scales, zeros, xx, out_dtype=torch.float32).cpu()
        b = fn(codes, scales, zeros, xx, out_dtype=torch.float32).cpu()
        assert torch.equal(a, b)


def test_end_to_end_quantize_then_gemv():
    # GPU quantizer output feeds the GPU GEMV; the oracle does both steps itself.
    wl = workloads.WORKLOADS["llama7b"]
    w, _ = workloads.weight(wl, 1)
    x = workloads.activations(wl, 1, w.shape[1])
    note("end-to-end quantize + gemv 11008x4096")
    codes, scales, zeros = qmm.quantize_groupwise(w.to(DEV))
    y = qmm.w4a16_gemv(codes, scales, zeros, x.to(DEV), out_dtype=torch.float32)
    q, s, z = oracle.asym_quantize(w.float().numpy())
    assert_close(y.cpu(), oracle.w4a16_reference(x.float().numpy(), q, s, z), "end-to-end")
