"""The Python binding checks every operand before it reaches the C ABI: a
mismatched shape, dtype, K or output raises ValueError on the host, before any
launch (these run on the CPU: shapes and dtypes are checked before the device,
so CPU tensors reach exactly the check under test)."""
import pytest
import torch

import quantized_matmul_quantize_amd as qmm

u8, f32, bf16, f16, i8 = torch.uint8, torch.float32, torch.bfloat16, torch.float16, torch.int8


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def fmt(N=8, K=256, bits=4, sdt=f32, group=128):
    G = K // group
    zc = (G + 1) // 2 if bits <= 4 else G
    return t((N, K * bits // 8), u8), t((N, G), sdt), t((N, zc), u8)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_gemv_checks():
    c, s, z = fmt()
    raises(lambda: qmm.w4a16_gemv(c, s, z, t((1, 128), bf16)), "x has shape")            # K mismatch
    raises(lambda: qmm.w4a16_gemv(c, s, z, t((1, 256), f32)), "x has dtype")              # fp32 activations
    raises(lambda: qmm.w4a16_gemv(c, s, z, t((9, 256), bf16)), "1 to 8 tokens")           # 9 tokens
    raises(lambda: qmm.w4a16_gemv(c, t((8, 3), f32), z, t((1, 256), bf16)), "scales has shape")
    raises(lambda: qmm.w4a16_gemv(c, s.half(), z, t((1, 256), bf16)), "scales has dtype")
    raises(lambda: qmm.w4a16_gemv(c, s, t((8, 2), u8), t((1, 256), bf16)), "zeros has shape")
    raises(lambda: qmm.w4a16_gemv(c.to(i8), s, z, t((1, 256), bf16)), "codes has dtype")
    raises(lambda: qmm.w4a16_gemv(c, s, z, t((1, 256), bf16)), "device tensor")          # all right but on CPU


def test_gemm_and_format_checks():
    c, s, z = fmt()
    raises(lambda: qmm.w4a16_gemm(c, s, z, t((4, 255), bf16)), "X has shape")
    raises(lambda: qmm.w4a16_gemm(c, s, z, t((4, 256), bf16), group=96), "not a multiple")
    c3, s3, z3 = fmt(bits=3, sdt=f16, group=32)
    raises(lambda: qmm.wxa16_gemv(c3, s3, z3, t((1, 256), bf16), group=32, bits=4), "has shape")  # bits disagree
    raises(lambda: qmm.wxa16_gemm(c3, s3, z3, t((4, 256), bf16), group=64, bits=3), "scales has shape")
    raises(lambda: qmm.wxa16_gemv(c3, s3.to(bf16), z3, t((1, 256), bf16), group=32, bits=3), "scale_dtype")
    raises(lambda: qmm.dequantize_ex(c3, s3, t((8, 8), u8), group=32, bits=3), "zeros has shape")
    c8, s8, z8 = fmt(bits=8)
    raises(lambda: qmm.dequantize(c8, s8, t((8, 1), u8), bits=8), "zeros has shape")       # 8 bits: a byte per group
    raises(lambda: qmm.quantize_groupwise(t((4, 200), bf16)), "not a multiple")
    raises(lambda: qmm.quantize_groupwise_ex(t((4, 256), bf16), bits=5), "bits")
    raises(lambda: qmm.quantize_groupwise_ex(t((4, 256), bf16), scale_dtype=bf16), "scale_dtype")
    raises(lambda: qmm.quantize_groupwise(t((4, 256), i8)), "W has dtype")


def test_output_checks():
    c, s, z = fmt()
    x = t((2, 256), bf16)
    raises(lambda: qmm.w4a16_gemv(c, s, z, x, out=t((2, 7), bf16)), "x|out")
    raises(lambda: qmm.dequantize(c, s, z, out=t((8, 256), f16)), "out has dtype|device")


def test_w8_and_w8a8_checks():
    raises(lambda: qmm.w8a16_gemv(t((8, 256), i8), t((7,), f32), t((1, 256), bf16)), "w_scale has shape")
    raises(lambda: qmm.w8a16_gemv(t((8, 256), u8), t((8,), f32), t((1, 256), bf16)), "qW has dtype")
    raises(lambda: qmm.sq_int8_gemm(t((4, 256), i8), t((4,), f32), t((8, 128), i8), t((8,), f32)), "qW has shape")
    raises(lambda: qmm.sq_int8_gemm(t((4, 256), i8), t((3,), f32), t((8, 256), i8), t((8,), f32)), "x_scale")
    raises(lambda: qmm.sq_smooth_factors(t((4, 256), bf16), t((8, 128), bf16)), "W has shape")
    raises(lambda: qmm.sq_quantize_weight(t((8, 256), bf16), t((128,), f32)), "smooth has shape")
    raises(lambda: qmm.smooth_quant_w8a8_gemm(t((4, 256), bf16), None, t((8, 256), i8), t((4,), f32)),
           "w_scale has shape")
    raises(lambda: qmm.smooth_quant_w8a8_gemm_noalloc(t((4, 256), bf16), t((256,), f16), t((8, 256), i8),
                                                      t((8,), f32)), "smooth has dtype")


def test_llm_int8_checks():
    x = t((4, 256), bf16)
    raises(lambda: qmm.llm_int8_gemm(t((4, 256), f32), t((8, 256), i8), t((8,), f32)), "X has dtype")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 128), i8), t((8,), f32)), "qW has shape")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), threshold=-1.0), "threshold")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), threshold=float("nan")), "threshold")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), max_outliers=-2), "max_outliers")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), out_dtype=torch.float16), "out_dtype")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), n_outliers=t((2,), f32)), "n_outliers")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32), workspace=t((16,), u8)), "workspace holds")
    raises(lambda: qmm.llm_int8_gemm(x, t((8, 256), i8), t((8,), f32)), "device tensor")
    raises(lambda: qmm.llm_int8_outliers(t((4, 256), f16), threshold=-0.5), "threshold")


def test_awq_checks():
    w, x = t((8, 256), bf16), t((4, 256), bf16)
    raises(lambda: qmm.awq_search(t((8, 256), f32), x), "W has dtype")
    raises(lambda: qmm.awq_search(t((8, 256), f16), x), "X has dtype")          # two 16-bit types
    raises(lambda: qmm.awq_search(w, t((4, 128), bf16)), "X has shape")
    raises(lambda: qmm.awq_search(t((8, 200), bf16), t((4, 200), bf16)), "multiple of 128")
    raises(lambda: qmm.awq_search(w, x, alphas=[]), "1 to 64 alphas")
    raises(lambda: qmm.awq_search(w, x, alphas=[0.1] * 65), "1 to 64 alphas")
    raises(lambda: qmm.awq_search(w, x, alphas=[0.5, 1.5]), r"\[0, 1\]")
    raises(lambda: qmm.awq_search(w, x, alphas=[float("nan")]), r"\[0, 1\]")
    raises(lambda: qmm.awq_search(w, x, workspace=t((16,), u8)), "workspace holds")
    raises(lambda: qmm.awq_search(w, x), "device tensor")


def test_awq_default_grid_is_the_listings():
    # numpy's linspace(0, 1, 11) values, to the last bit (0.30000000000000004 ...)
    import numpy as np
    assert np.array_equal(np.array(qmm.AWQ_ALPHAS), np.linspace(0.0, 1.0, 11))
