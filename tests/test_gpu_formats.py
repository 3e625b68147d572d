"""GPU parity for the stored-format variants (group sizes 32..1024, 3-, 4- and
8-bit codes, binary16 scales, both grids): quantizer and dequantizer bit for
bit against the CPU oracle, GEMV / GEMM within the elementwise tolerance; and
the 4-bit repack between plain nibble order and the library's code words."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import assert_close, bits_equal, first_diff, note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
SDT = {"s32": torch.float32, "s16": torch.float16}


def _weights(shape, dtype, seed, outliers=True):
    g = workloads.rng(77, seed)
    w = workloads.gaussian(g, shape, 0.02)
    if outliers:
        workloads.plant_scale_entries(w, g, 0.002, 10.0)
    w[0, :64] = 0.0                                     # all-zero runs (s = 1 for small groups)
    w[-1, -256:] = np.abs(w[-1, -256:])                 # one-signed groups
    return workloads.to_dtype(w, dtype)


def _gpu_format(w_cpu, group, bits, sdt, sym):
    codes, scales, zeros = qmm.quantize_groupwise_ex(w_cpu.to(DEV), group, bits, sdt, sym)
    torch.cuda.synchronize()
    return codes, scales, zeros


def _compare_format(w_cpu, group, bits, sdt, sym, what):
    note(f"quantize_groupwise_ex {what} shape={tuple(w_cpu.shape)} {w_cpu.dtype} group={group} bits={bits} "
         f"scales={sdt} sym={sym}")
    codes, scales, zeros = _gpu_format(w_cpu, group, bits, sdt, sym)
    q, s, z = oracle.quantize_format(w_cpu.float().numpy(), group, bits, sym, sdt == torch.float16)
    rc, rs, rz = oracle.pack_format(q, s, z, bits, sdt == torch.float16)
    c, sg, zg = codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy()
    assert bits_equal(sg, rs), f"{what} scales: {first_diff(sg, rs)}"
    assert bits_equal(zg, rz), f"{what} zeros: {first_diff(zg, rz)}"
    assert bits_equal(c, rc), f"{what} codes: {first_diff(c, rc)}"
    return (codes, scales, zeros), (q, s, z)


@pytest.mark.parametrize("sym", [False, True], ids=["asym", "sym"])
@pytest.mark.parametrize("sdt", ["s32", "s16"])
@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("group", [32, 64, 128, 256, 1024])
def test_quantize_dequantize_formats(group, bits, sdt, sym):
    shape = (67, 3072) if group != 1024 else (33, 3072)     # 3 groups of 1024: an odd count per row
    w = _weights(shape, "bf16", group * 10 + bits)
    (codes, scales, zeros), (q, s, z) = _compare_format(w, group, bits, SDT[sdt], sym, "small")
    ref = oracle.asym_dequantize(q, s, z, group)
    for odt in ("f32", "bf16"):
        note(f"dequantize_ex group={group} bits={bits} scales={sdt} out={odt}")
        out = qmm.dequantize_ex(codes, scales, zeros, TDT[odt], group, bits)
        torch.cuda.synchronize()
        want = ref if odt == "f32" else torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
        got = out.float().cpu().numpy()
        assert bits_equal(got.astype(np.float32), want.astype(np.float32)), f"dequantize_ex: {first_diff(got, want)}"


@pytest.mark.parametrize("wdt", ["f32", "f16"])
@pytest.mark.parametrize("bits", [3, 8])
def test_quantize_formats_input_dtypes(wdt, bits):
    w = _weights((40, 2048), wdt, 5 + bits)
    _compare_format(w, 64, bits, torch.float16, False, f"input-{wdt}")


def test_f16_scale_saturation_and_underflow():
    # ranges whose 16-bit scale rounds to 0 (stored as 1) or saturates at 65504
    w = np.zeros((4, 256), np.float32)
    w[0, :128] = np.linspace(-1e-8, 1e-8, 128)
    w[1, :128] = np.linspace(-2e6, 1e5, 128)
    w[2, :128] = np.linspace(0, 5e6, 128)
    w[3] = np.random.Generator(np.random.PCG64(3)).standard_normal(256) * 0.02
    for sym in (False, True):
        _compare_format(torch.from_numpy(w), 128, 4, torch.float16, sym, "extreme-ranges")


def test_old_entry_points_take_other_formats():
    # quantize_groupwise / dequantize / w4a16_gemv with group 64: the stored
    # format with fp32 scales, identical to the _ex calls
    w = _weights((96, 2048), "bf16", 11)
    wd = w.to(DEV)
    a = qmm.quantize_groupwise(wd, group=64)
    b = qmm.quantize_groupwise_ex(wd, 64, 4, torch.float32, False)
    x = workloads.activations(workloads.WORKLOADS["llama7b"], 1, 2048).to(DEV)
    ya = qmm.w4a16_gemv(*a, x, out_dtype=torch.float32, group=64)
    yb = qmm.wxa16_gemv(*b, x, out_dtype=torch.float32, group=64, bits=4)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.cpu(), v.cpu())
    assert torch.equal(ya.cpu(), yb.cpu())
    c8 = qmm.quantize_groupwise(wd, group=128, bits=8)
    r8 = qmm.quantize_groupwise_ex(wd, 128, 8, torch.float32, False)
    for u, v in zip(c8, r8):
        assert torch.equal(u.cpu(), v.cpu())


def _mm_reference(x_cpu, q, s, z, group):
    return oracle.w4a16_reference(x_cpu.float().numpy(), q, s, z, group)


@pytest.mark.parametrize("sdt", ["s32", "s16"])
@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("group", [32, 128, 1024])
@pytest.mark.parametrize("B", [1, 2, 3, 8])
def test_gemv_formats(B, group, bits, sdt):
    shape = (1000, 4096)
    w = _weights(shape, "bf16", B * 100 + group + bits)
    (codes, scales, zeros), (q, s, z) = _compare_format(w, group, bits, SDT[sdt], False, "gemv")
    x = workloads.activations(workloads.WORKLOADS["mlp70b"], B, shape[1], salt=bits)
    ref = _mm_reference(x, q, s, z, group)
    for xdt in ("bf16", "f16"):
        note(f"wxa16_gemv B={B} group={group} bits={bits} scales={sdt} x={xdt}")
        xd = x.to(TDT[xdt]).to(DEV)
        refx = _mm_reference(x.to(TDT[xdt]), q, s, z, group) if xdt == "f16" else ref
        y32 = qmm.wxa16_gemv(codes, scales, zeros, xd, out_dtype=torch.float32, group=group, bits=bits)
        y16 = qmm.wxa16_gemv(codes, scales, zeros, xd, group=group, bits=bits)
        torch.cuda.synchronize()
        assert_close(y32, refx, f"gemv B={B} g={group} b={bits} {sdt} {xdt} f32")
        assert_close(y16, refx, f"gemv B={B} g={group} b={bits} {sdt} {xdt} {xdt}")


@pytest.mark.parametrize("sdt", ["s32", "s16"])
@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("group", [32, 64, 256, 1024])
@pytest.mark.parametrize("M", [16, 77])
def test_gemm_formats(M, group, bits, sdt):
    shape = (300, 2048)
    w = _weights(shape, "bf16", M + group + bits)
    (codes, scales, zeros), (q, s, z) = _compare_format(w, group, bits, SDT[sdt], True, "gemm")
    X = workloads.activations(workloads.WORKLOADS["gemm"], M, shape[1], salt=group)
    ref = _mm_reference(X, q, s, z, group)
    note(f"wxa16_gemm M={M} group={group} bits={bits} scales={sdt}")
    Y = qmm.wxa16_gemm(codes, scales, zeros, X.to(DEV), out_dtype=torch.float32, group=group, bits=bits)
    Yb = qmm.wxa16_gemm(codes, scales, zeros, X.to(DEV), group=group, bits=bits)
    torch.cuda.synchronize()
    assert_close(Y, ref, f"gemm M={M} g={group} b={bits} {sdt}")
    assert_close(Yb, ref, f"gemm M={M} g={group} b={bits} {sdt} bf16")


@pytest.mark.parametrize("case", ["g128-4bit-f16scale", "g32-4bit", "g1024-4bit", "g128-3bit", "g128-8bit"])
def test_formats_full_size(case):
    # the 70B-class 28672 x 8192 matrix: every code, scale and zero-point bit
    # for bit; the B=1 GEMV on every row and the B=8 GEMV on rows covering
    # every block of 8 rows in a stride
    group, bits, sdt = {"g128-4bit-f16scale": (128, 4, torch.float16), "g32-4bit": (32, 4, torch.float32),
                        "g1024-4bit": (1024, 4, torch.float32), "g128-3bit": (128, 3, torch.float16),
                        "g128-8bit": (128, 8, torch.float16)}[case]
    wl = workloads.WORKLOADS["mlp70b"]
    w, _ = workloads.weight(wl, 0)
    (codes, scales, zeros), (q, s, z) = _compare_format(w, group, bits, sdt, False, f"mlp70b[0] {case}")
    del w
    x1 = workloads.activations(wl, 1, 8192, salt=0)
    note(f"wxa16_gemv B=1 full size {case}")
    y1 = qmm.wxa16_gemv(codes, scales, zeros, x1.to(DEV), out_dtype=torch.float32, group=group, bits=bits)
    torch.cuda.synchronize()
    assert_close(y1, _mm_reference(x1, q, s, z, group), f"full-size B=1 {case}")
    x8 = workloads.activations(wl, 8, 8192, salt=0)
    rows = np.unique(np.concatenate([np.arange(0, 28672, 61), np.arange(28672 - 64, 28672)]))
    note(f"wxa16_gemv B=8 full size {case}")
    y8 = qmm.wxa16_gemv(codes, scales, zeros, x8.to(DEV), out_dtype=torch.float32, group=group, bits=bits)
    torch.cuda.synchronize()
    ref8 = _mm_reference(x8, q[rows], s[rows], z[rows], group)
    assert_close(y8.cpu()[:, torch.from_numpy(rows)], ref8, f"full-size B=8 {case}")


@pytest.mark.parametrize("shape", [(3, 16), (64, 1024), (129, 2176), (1000, 4104)])
def test_repack_plain_order(shape):
    # plain nibble order (the oracle's pack_nibbles) -> code words equal the
    # oracle's pack_codes; back again; and in place
    g = np.random.Generator(np.random.PCG64(shape[0]))
    q = g.integers(0, 16, size=shape).astype(np.uint8)
    plain = oracle.pack_nibbles(q)
    words = oracle.pack_codes(q)
    note(f"w4_repack shape={shape}")
    p_dev = torch.from_numpy(plain).to(DEV)
    c = qmm.w4_repack_from_plain(p_dev)
    back = qmm.w4_repack_to_plain(c)
    inplace = p_dev.clone()
    qmm.lib().qmm_w4_repack_from_plain(qmm._ptr(inplace), qmm._ptr(inplace), shape[0], shape[1], qmm._stream(inplace))
    torch.cuda.synchronize()
    assert bits_equal(c.cpu().numpy(), words), first_diff(c.cpu().numpy(), words)
    assert bits_equal(back.cpu().numpy(), plain)
    assert bits_equal(inplace.cpu().numpy(), words)


def test_repack_then_gemv():
    # weights packed in plain nibble order go through the repack and then the
    # library's GEMV, matching the oracle's product
    w, _ = workloads.weight(workloads.WORKLOADS["llama7b"], 0, shape=(512, 4096))
    q, s, z = oracle.asym_quantize(w.float().numpy())
    plain = torch.from_numpy(oracle.pack_nibbles(q)).to(DEV)
    x = workloads.activations(workloads.WORKLOADS["llama7b"], 1, 4096)
    note("repack_from_plain -> w4a16_gemv 512x4096")
    codes = qmm.w4_repack_from_plain(plain)
    y = qmm.w4a16_gemv(codes, torch.from_numpy(s).to(DEV), torch.from_numpy(oracle.pack_nibbles(z)).to(DEV),
                       x.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(y, oracle.w4a16_reference(x.float().numpy(), q, s, z), "repack + gemv")
