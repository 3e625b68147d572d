"""C-ABI checks that need no GPU: every declared symbol is exported, the host-only
entry points compute what they state, and argument errors are reported before
any HIP call (no kernel is ever launched from here: every call below fails
validation, and the fake device pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_matmul_quantize_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

OK, EINVAL, EUNSUP, EALIGN, EWS, EHIP, ERANGE = 0, -1, -2, -3, -4, -5, -6
P = 0x7F0000000000          # 16-byte aligned stand-in for a device pointer
MIS = P + 2                 # misaligned
BF16, F16, F32, I32 = qmm.BF16, qmm.F16, qmm.F32, qmm.I32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["quantize_groupwise", "dequantize", "w4a16_gemv", "w4a16_gemm", "smooth_quant_w8a8_gemm"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(qmm.library_path)
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", qmm.library_path], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    for n in names:
        assert n in exported, f"{n} is not an unmangled exported symbol"


def test_binding_covers_every_symbol():
    assert set(declared_functions()) <= set(qmm._SIGS)


def test_binding_names_match_the_header():
    # every C entry point has a Python function of the same name, and every
    # name the package exports resolves
    for n in declared_functions():
        if n in ("qmm_status_string", "qmm_version", "sq_workspace_bytes"):
            continue
        py = n[4:] if n.startswith("qmm_") else n
        assert callable(getattr(qmm, py, None)), n
    for n in qmm.__all__:
        assert hasattr(qmm, n), n


def test_w8a16_argument_errors():
    f = qmm.lib().w8a16_gemv
    assert f(None, P, 8, 256, P, BF16, 1, P, BF16, None) == EINVAL
    assert f(P, P, 0, 256, P, BF16, 1, P, BF16, None) == EINVAL
    assert f(P, P, 8, 256, P, BF16, 0, P, BF16, None) == EINVAL
    assert f(P, P, 8, 256, P, BF16, 9, P, BF16, None) == EUNSUP     # B > 8
    assert f(P, P, 8, 200, P, BF16, 1, P, BF16, None) == EUNSUP     # K % 64
    assert f(P, P, 8, 256, P, F32, 1, P, F32, None) == EUNSUP       # fp32 activations
    assert f(P, P, 8, 256, P, BF16, 1, P, F16, None) == EUNSUP      # mixed 16-bit types
    assert f(P, P, 8, 256, P, 7, 1, P, BF16, None) == EINVAL        # bad dtype value
    assert f(P, P, 8, (1 << 24) + 64, P, BF16, 1, P, BF16, None) == ERANGE
    assert f(P, P, 8, 256, MIS, BF16, 1, P, BF16, None) == EALIGN


def test_status_strings_and_version():
    lib = qmm.lib()
    for st in [OK, EINVAL, EUNSUP, EALIGN, EWS, EHIP, ERANGE, -99]:
        assert lib.qmm_status_string(st)
    assert lib.qmm_status_string(EALIGN).startswith(b"QMM_EALIGN")
    assert lib.qmm_version() >= 10000


def test_w4_sizes():
    assert qmm.w4_sizes(28672, 8192) == (28672 * 4096, 28672 * 64 * 4, 28672 * 32)
    assert qmm.w4_sizes(3, 384) == (3 * 192, 3 * 3 * 4, 3 * 2)
    with pytest.raises(qmm.QmmError):
        qmm.w4_sizes(4, 100)
    lib = qmm.lib()
    assert lib.qmm_w4_sizes(0, 128, 128, None, None, None) == EINVAL
    assert lib.qmm_w4_sizes(4, 128, 0, None, None, None) == EINVAL


def test_w4_sizes_match_storage_example():
    # 0.5 B per weight + per-group scale and 4-bit zero-point; with the page's
    # 16-bit scale a 70B model is ~36.4 GB ("How quantization works", Exercises 2).
    n, k = 8192, 8192
    c, s, z = qmm.w4_sizes(n, k)
    per_param_fp16_scale = (c + s / 2 + z) / (n * k)
    assert abs(70e9 * per_param_fp16_scale / 1e9 - 36.4) < 0.05


def test_sq_workspace_bytes():
    lib = qmm.lib()
    assert lib.sq_workspace_bytes(2048, 4096) == 2048 * 4096 + 2048 * 4
    assert lib.sq_workspace_bytes(3, 64) == 256 + 12
    assert lib.sq_workspace_bytes(0, 64) == 0


def test_quantize_argument_errors():
    f = qmm.lib().quantize_groupwise
    assert f(None, BF16, 4, 256, 128, 4, P, P, P, None) == EINVAL
    assert f(P, BF16, 4, 256, 128, 4, None, P, P, None) == EINVAL
    assert f(P, BF16, 0, 256, 128, 4, P, P, P, None) == EINVAL
    assert f(P, BF16, 4, 200, 128, 4, P, P, P, None) == EINVAL          # K % group
    assert f(P, 9, 4, 256, 128, 4, P, P, P, None) == EINVAL             # bad dtype
    assert f(P, I32, 4, 256, 128, 4, P, P, P, None) == EUNSUP
    assert f(P, BF16, 4, 256, 128, 5, P, P, P, None) == EUNSUP          # bits
    assert f(P, BF16, 4, 4096, 2048, 4, P, P, P, None) == EUNSUP        # group
    assert f(MIS, BF16, 4, 256, 128, 4, P, P, P, None) == EALIGN
    assert f(P, BF16, 4, 256, 128, 4, MIS, P, P, None) == EALIGN


def test_dequantize_argument_errors():
    f = qmm.lib().dequantize
    assert f(P, P, P, 4, 256, 128, 4, None, F32, None) == EINVAL
    assert f(P, P, P, 4, 256, 128, 4, P, I32, None) == EUNSUP
    assert f(P, P, P, 4, 256, 128, 4, MIS, F32, None) == EALIGN
    assert f(P, P, P, -1, 256, 128, 4, P, F32, None) == EINVAL


def test_gemv_gemm_argument_errors():
    gemv = qmm.lib().w4a16_gemv
    gemm = qmm.lib().w4a16_gemm
    assert gemv(P, P, P, 8, 256, 128, None, BF16, 1, P, BF16, None) == EINVAL
    assert gemv(P, P, P, 8, 256, 128, P, BF16, 9, P, BF16, None) == EUNSUP    # B > 8
    assert gemv(P, P, P, 8, 256, 128, P, BF16, 0, P, BF16, None) == EINVAL
    assert gemv(P, P, P, 8, 256, 128, P, F32, 1, P, F32, None) == EUNSUP      # fp32 activations
    assert gemv(P, P, P, 8, 256, 128, P, BF16, 1, P, F16, None) == EUNSUP     # mixed 16-bit types
    assert gemv(P, P, P, 8, 256, 256, P, BF16, 9, P, BF16, None) == EUNSUP   # B > 8, other group
    assert gemv(P, P, P, 8, 4096, 2048, P, BF16, 1, P, BF16, None) == EUNSUP # group
    assert gemv(P, P, P, 8, 256, 128, MIS, BF16, 1, P, BF16, None) == EALIGN
    assert gemm(P, P, P, 8, 256, 128, P, F32, 4, P, F32, None) == EUNSUP      # fp32 activations
    assert gemm(P, P, P, 8, 256, 128, P, F16, 4, P, BF16, None) == EUNSUP     # mixed 16-bit types
    assert gemm(P, P, P, 8, 300, 128, P, BF16, 4, P, BF16, None) == EINVAL
    assert gemm(P, P, P, 8, 256, 128, P, BF16, 0, P, BF16, None) == EINVAL
    assert gemv(P, P, P, 8, (1 << 24) + 128, 128, P, BF16, 1, P, BF16, None) == ERANGE   # K past 2^24
    assert gemm(P, P, P, 1 << 31, 256, 128, P, BF16, 4, P, BF16, None) == ERANGE


def test_w8a8_argument_errors():
    lib = qmm.lib()
    assert lib.sq_int8_gemm(P, P, P, P, 4, 4, 131072, P, BF16, None) == ERANGE   # int32 bound
    assert lib.sq_int8_gemm(P, P, P, P, 4, 4, 131136, P, BF16, None) == ERANGE
    assert lib.sq_int8_gemm(P, P, P, P, 4, 4, 100, P, BF16, None) == EUNSUP      # K % 64
    assert lib.sq_int8_gemm(P, None, P, P, 4, 4, 128, P, BF16, None) == EINVAL   # scale needed
    assert lib.sq_int8_gemm(P, P, P, P, 4, 4, 128, P, F16, None) == EUNSUP
    assert lib.sq_int8_gemm(MIS, P, P, P, 4, 4, 128, P, I32, None) == EALIGN
    assert lib.sq_quantize_weight(P, BF16, None, 4, 100, P, P, None) == EUNSUP
    assert lib.sq_quantize_weight(P, I32, None, 4, 128, P, P, None) == EUNSUP
    assert lib.sq_quantize_activation(None, BF16, None, 4, 128, P, P, None) == EINVAL
    assert lib.sq_quantize_activation(P, BF16, P + 1, 4, 128, P, P, None) == EALIGN
    assert lib.sq_smooth_factors(P, BF16, 4, P, BF16, 4, 128, ctypes.c_float(1.5), P, P, P, None) == EINVAL
    assert lib.sq_smooth_factors(P, BF16, 4, P, BF16, 4, 100, ctypes.c_float(0.5), P, P, P, None) == EUNSUP
    sq = lib.smooth_quant_w8a8_gemm
    need = lib.sq_workspace_bytes(4, 128)
    assert sq(P, BF16, None, P, P, 4, 4, 128, P, BF16, None, need, None) == EWS
    assert sq(P, BF16, None, P, P, 4, 4, 128, P, BF16, P, need - 1, None) == EWS
    assert sq(P, BF16, None, P, P, 4, 4, 128, P, BF16, MIS, need, None) == EWS
    assert sq(P, BF16, None, P, P, 4, 4, 131136, P, BF16, P, 10**9, None) == ERANGE


def test_llm_int8_workspace_and_argument_errors():
    lib = qmm.lib()
    ws = lib.llm_int8_workspace_bytes
    # X_q, token scales, factors, index list, counts (each at a 256-byte boundary)
    assert ws(2048, 4096, 4096, 64) == 2048 * 4096 + 2048 * 4 + 4096 * 4 + 256 + 256
    assert ws(3, 5, 64, 2) == 256 * 5
    assert ws(2048, 4096, 4096, 4096) == 2048 * 4096 + 2048 * 4 + 4096 * 4 + 4096 * 4 + 256
    assert ws(4, 8, 128, 10**6) == ws(4, 8, 128, 128)                  # the cap is at most K
    assert ws(0, 8, 128, 4) == 0 and ws(4, 8, 128, -1) == 0
    g = lib.llm_int8_gemm
    need = ws(4, 8, 128, 8)
    f = ctypes.c_float
    args = lambda **k: [k.get("X", P), k.get("xdt", BF16), P, P, 4, 8, k.get("K", 128), f(k.get("tau", 6.0)),
                        k.get("cap", 8), k.get("Y", P), k.get("ydt", BF16), None, k.get("ws", P),
                        k.get("wsb", need), None]
    assert g(*args(X=None)) == EINVAL
    assert g(*args(xdt=F32)) == EUNSUP
    assert g(*args(xdt=I32)) == EINVAL
    assert g(*args(ydt=F16)) == EUNSUP
    assert g(*args(ydt=I32)) == EUNSUP
    assert g(*args(tau=-1.0)) == EINVAL
    assert g(*args(tau=float("nan"))) == EINVAL
    assert g(*args(cap=-1)) == EINVAL
    assert g(*args(K=100)) == EUNSUP
    assert g(*args(K=131136, wsb=10**12)) == ERANGE
    assert g(*args(X=MIS)) == EALIGN
    assert g(*args(ws=None)) == EWS
    assert g(*args(wsb=need - 1)) == EWS
    assert g(*args(ws=MIS)) == EWS
    o = lib.llm_int8_outliers
    assert o(P, BF16, 4, 128, f(6.0), 8, None, P, P, None) == EINVAL
    assert o(P, F32, 4, 128, f(6.0), 8, P, P, P, None) == EUNSUP
    assert o(P, BF16, 4, 128, f(6.0), 8, P + 2, P, P, None) == EALIGN


def test_binding_raises_qmm_error():
    with pytest.raises(qmm.QmmError) as e:
        qmm._call("sq_int8_gemm", P, P, P, P, 4, 4, 131136, P, BF16, None)
    assert e.value.status == ERANGE
    assert "QMM_ERANGE" in str(e.value)


def test_awq_workspace_and_argument_errors():
    lib = qmm.lib()
    ws = lib.awq_workspace_bytes
    a256 = lambda b: (b + 255) // 256 * 256
    # magnitude partial sums (32-row slices), the magnitudes, every alpha's
    # fp64 powers, their per-256-column maxima and minima, the norms, the fp32
    # factors, the chosen factors, the scaled bf16 inputs and their per-group
    # sums, one INT4 format, both fp32 products, the squared-error partial sums
    n, k, t, na = 4096, 4096, 2048, 11
    want = (a256(64 * k * 8) + a256(k * 8) + a256(na * k * 8) + 2 * a256(na * 16 * 8) + a256(na * 8) + a256(na * k * 4) +
            a256(k * 4) + a256(t * k * 2) + a256(t * 32 * 4) + a256(n * k // 2) + a256(n * 32 * 4) + a256(n * 16) +
            2 * a256(t * n * 4) + a256(na * 1024 * 8))
    assert ws(n, k, t, na) == want
    assert ws(0, 128, 4, 1) == 0 and ws(4, 100, 4, 1) == 0 and ws(4, 128, 4, 65) == 0 and ws(4, 128, 4, 0) == 0
    g = lib.awq_search
    need = ws(4, 128, 4, 2)
    al = (ctypes.c_double * 2)(0.0, 1.0)
    bad = (ctypes.c_double * 2)(0.0, 1.5)
    args = lambda **k: [k.get("W", P), k.get("wdt", BF16), P, k.get("xdt", BF16), 4, k.get("K", 128), 4,
                        k.get("al", ctypes.cast(al, ctypes.c_void_p)), k.get("na", 2), P, P, P, P, P, P,
                        k.get("ws", P), k.get("wsb", need), None]
    assert g(*args(W=None)) == EINVAL
    assert g(*args(wdt=F16)) == EUNSUP                                   # bf16 X with fp16 W
    assert g(*args(wdt=F32, xdt=F32)) == EUNSUP
    assert g(*args(xdt=F32)) == EUNSUP
    assert g(*args(wdt=I32)) == EINVAL
    assert g(*args(K=100)) == EUNSUP
    assert g(*args(na=65)) == EUNSUP
    assert g(*args(na=0)) == EINVAL
    assert g(*args(al=ctypes.cast(bad, ctypes.c_void_p))) == EINVAL
    assert g(*args(K=(1 << 22) + 128, wsb=10**15)) == ERANGE
    assert g(P, BF16, P, BF16, 4, 128, 65535 * 32 + 1, ctypes.cast(al, ctypes.c_void_p), 2, P, P, P, P, P, P,
             P, 10**15, None) == ERANGE
    assert g(*args(W=MIS)) == EALIGN
    assert g(*args(ws=None)) == EWS
    assert g(*args(wsb=need - 1)) == EWS
    assert g(*args(ws=MIS)) == EALIGN
