"""CPU oracle for the quantizer and the quantized matmuls -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It wraps ``qmm_oracle.c`` (plain single-threaded C loops, IEEE fp32
where the method is fp32, fp64 sums for matmul references) with numpy
marshalling.  It imports nothing from the HIP library and the HIP library
imports nothing from it.

Each function names the passage it follows; the C file carries the full list
of sources and of the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB = os.path.join(_HERE, "libqmm_oracle.so")
_LIB_OMP = os.path.join(_HERE, "libqmm_oracle_omp.so")

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99", "-Wall",
             "-Wno-unknown-pragmas"]


def build(force: bool = False, parallel: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math).
    parallel=True builds the timing-only variant with the row loops of the
    dequantizer and the matmul reference split over OpenMP threads.  A
    library older than the source is rebuilt."""
    path = _LIB_OMP if parallel else _LIB
    if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        tmp = path + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, *(["-fopenmp"] if parallel else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, path)
    return path


_lib = None
_lib_omp = None


def lib(parallel: bool = False) -> ctypes.CDLL:
    """The oracle library; parallel=True the OpenMP build (timing only)."""
    global _lib, _lib_omp
    if (_lib_omp if parallel else _lib) is None:
        l = ctypes.CDLL(build(parallel=parallel))
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        F = ctypes.c_float
        sigs = {
            "oq_asym_quantize": [P, I64, I64, I64, I, P, P, P],
            "oq_asym_dequantize": [P, P, P, I64, I64, I64, P],
            "oq_sym_quantize": [P, I64, I64, I64, I, F, P, P],
            "oq_sym_dequantize": [P, P, I64, I64, I64, P],
            "oq_pack_nibbles": [P, I64, I64, P],
            "oq_pack_codes": [P, I64, I64, P],
            "oq_matmul_nt_f64": [P, P, I64, I64, I64, P],
            "oq_int8_matmul_nt": [P, P, I64, I64, I64, P],
            "oq_rescale_f64": [P, P, P, I64, I64, P],
            "oq_col_absmax": [P, I64, I64, P],
            "oq_smooth_factors": [P, P, I64, F, P],
            "oq_scale_columns_mul": [P, P, I64, I64, P],
            "oq_scale_columns_div": [P, P, I64, I64, P],
            "oq_threads": [],
            "oq_quantize_format": [P, I64, I64, I64, I, I, I, P, P, P],
            "oq_pack_codes3": [P, I64, I64, P],
            "oq_f32_to_f16_array": [P, I64, P],
            "oq_f16_to_f32_array": [P, I64, P],
            "oq_e4m3_array": [P, I64, P],
            "oq_e4m3_decode_array": [P, I64, P],
            "oq_fp8_quantize": [P, I64, I64, I64, P, P],
            "oq_fp8_matmul_nt": [P, P, I64, I64, I64, P],
            "oq_llm_int8": [P, I64, I64, P, P, I64, F, I64, I, P, P, P, P, P],
            "oq_awq_search": [P, P, I64, I64, I64, P, I64, P, P, P, P, P, P, I],
            "oq_awq_factors": [P, I64, I64, P, I64, P],
        }
        for name, argtypes in sigs.items():
            fn = getattr(l, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        if parallel:
            _lib_omp = l
        else:
            _lib = l
    return _lib_omp if parallel else _lib


def _p(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise ValueError(f"oracle {what} failed with status {status}")


# --------------------------------------------------------------------------
# Asymmetric group-wise quantization (s, z, codes) and its inverse.
# "Quantization Explained" slides "Scale and Zero-Point" / "Manual Group-Wise
# Quantizer"; "How quantization works", "The math of quantization".
# --------------------------------------------------------------------------
def asym_quantize(w, group: int = 128, bits: int = 4) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (codes uint8 [rows, cols] unpacked, scales f32 [rows, G], zeros uint8 [rows, G])."""
    w = _f32(w)
    if w.ndim == 1:
        w = w[None, :]
    rows, cols = w.shape
    if group <= 0 or cols % group:
        raise ValueError("cols must be a multiple of group")
    g = cols // group
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, g), np.float32)
    z = np.empty((rows, g), np.uint8)
    _check(lib().oq_asym_quantize(_p(w), rows, cols, group, bits, _p(q), _p(s), _p(z)), "asym_quantize")
    return q, s, z


def asym_dequantize(q, s, z, group: int = 128, parallel: bool = False) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s = _f32(s)
    z = np.ascontiguousarray(z, np.uint8)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float32)
    _check(lib(parallel).oq_asym_dequantize(_p(q), _p(s), _p(z), rows, cols, group, _p(out)), "asym_dequantize")
    return out


def pack_nibbles(vals) -> np.ndarray:
    """Row-wise two-per-byte packing (element 2j low nibble, 2j+1 high nibble)."""
    vals = np.ascontiguousarray(vals, np.uint8)
    if vals.ndim == 1:
        vals = vals[None, :]
    rows, count = vals.shape
    out = np.empty((rows, (count + 1) // 2), np.uint8)
    _check(lib().oq_pack_nibbles(_p(vals), rows, count, _p(out)), "pack_nibbles")
    return out


def pack_codes(vals) -> np.ndarray:
    """Row-wise code words: per run of 8 elements one little-endian 32-bit word,
    element 2i in bits 4i.., element 2i+1 in bits 16+4i.. (the layout of the
    library's weight codes; the pages fix only half a byte per weight)."""
    vals = np.ascontiguousarray(vals, np.uint8)
    if vals.ndim == 1:
        vals = vals[None, :]
    rows, count = vals.shape
    out = np.empty((rows, count // 2), np.uint8)
    _check(lib().oq_pack_codes(_p(vals), rows, count, _p(out)), "pack_codes")
    return out


def quantize_format(w, group: int = 128, bits: int = 4, symmetric: bool = False, scale_f16: bool = False):
    """Group-wise quantization in any of the stored formats (asymmetric or
    symmetric grid, bits in 2..8, fp32 or binary16 scales): returns (codes
    uint8 [rows, cols] unpacked, scales f32 [rows, G] holding the stored value,
    zeros uint8 [rows, G]).  "How quantization works", "The math of
    quantization" and Exercise 2 (16-bit scales); "Quantization Explained",
    "Scale and Zero-Point", "Manual Group-Wise Quantizer"."""
    w = _f32(w)
    if w.ndim == 1:
        w = w[None, :]
    rows, cols = w.shape
    if group <= 0 or cols % group:
        raise ValueError("cols must be a multiple of group")
    g = cols // group
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, g), np.float32)
    z = np.empty((rows, g), np.uint8)
    _check(lib().oq_quantize_format(_p(w), rows, cols, group, bits, int(symmetric), int(scale_f16), _p(q), _p(s),
                                    _p(z)), "quantize_format")
    return q, s, z


def f32_to_f16(a) -> np.ndarray:
    """IEEE binary16 of each float32 (round to nearest even, saturating at 65504), as np.float16."""
    a = _f32(a)
    out = np.empty(a.shape, np.uint16)
    _check(lib().oq_f32_to_f16_array(_p(a), a.size, _p(out)), "f32_to_f16")
    return out.view(np.float16)


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, np.float32)
    _check(lib().oq_f16_to_f32_array(_p(h), h.size, _p(out)), "f16_to_f32")
    return out


def pack_codes3(vals) -> np.ndarray:
    """3-bit codes in the library's layout: per run of 32 elements of a row, three little-endian words;
    element e < 30 in word e // 10 at bit 3 (r // 2) + 16 (r % 2), r = e % 10; bit t of element 30
    (31) at bit 15 (31) of word t."""
    vals = np.ascontiguousarray(vals, np.uint8)
    if vals.ndim == 1:
        vals = vals[None, :]
    rows, count = vals.shape
    out = np.empty((rows, count * 3 // 8), np.uint8)
    _check(lib().oq_pack_codes3(_p(vals), rows, count, _p(out)), "pack_codes3")
    return out


def pack_format(q, s, z, bits: int, scale_f16: bool):
    """Stored form of quantize_format's output: codes (4 bits: the code words
    of pack_codes; 8 bits: one byte each; 3 bits: pack_codes3), scales (float32
    or binary16) and zero-points (two per byte up to 4 bits, else one byte)."""
    q = np.ascontiguousarray(q, np.uint8)
    if bits == 4:
        codes = pack_codes(q)
    elif bits == 8:
        codes = q.copy()
    elif bits == 3:
        codes = pack_codes3(q)
    else:
        raise ValueError("stored formats have 3, 4 or 8 bits")
    scales = f32_to_f16(s) if scale_f16 else _f32(s).copy()
    zeros = pack_nibbles(z) if bits <= 4 else np.ascontiguousarray(z, np.uint8).copy()
    return codes, scales, zeros


def quantize_format_packed(w, group: int = 128, bits: int = 4, symmetric: bool = False, scale_f16: bool = False):
    """The stored format of any variant: (codes, scales, zeros) as pack_format."""
    q, s, z = quantize_format(w, group, bits, symmetric, scale_f16)
    return pack_format(q, s, z, bits, scale_f16)


def quantize_groupwise_packed(w, group: int = 128):
    """The stored INT4 format: (codes [N, K/2] u8, scales [N, G] f32, zeros [N, ceil(G/2)] u8)."""
    q, s, z = asym_quantize(w, group, 4)
    return pack_codes(q), s, pack_nibbles(z)


def sym_quantize_int4_packed(w, group: int = 128):
    """Symmetric INT4 per group ("How quantization works", "The math of
    quantization"; absmax floored at 1e-8 as in the INT8 path), stored in the
    same format as quantize_groupwise_packed: code q + 8 and zero-point 8.
    Returns (codes [N, K/2] u8, scales [N, G] f32, zeros [N, ceil(G/2)] u8,
    q int8 [N, K])."""
    q, s = sym_quantize(w, group, 4, 1e-8)
    z = np.full(s.shape, 8, np.uint8)
    return pack_codes((q.astype(np.int16) + 8).astype(np.uint8)), s, pack_nibbles(z), q


# --------------------------------------------------------------------------
# Symmetric quantization ("How quantization works", "The math of
# quantization" and the fake-quantization listing's 1e-8 absmax floor).
# --------------------------------------------------------------------------
def sym_quantize(x, group: int, bits: int = 8, floor: float = 1e-8) -> Tuple[np.ndarray, np.ndarray]:
    x = _f32(x)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    if group <= 0 or cols % group:
        raise ValueError("cols must be a multiple of group")
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, cols // group), np.float32)
    _check(lib().oq_sym_quantize(_p(x), rows, cols, group, bits, ctypes.c_float(floor), _p(q), _p(s)),
           "sym_quantize")
    return q, s


def sym_dequantize(q, s, group: int) -> np.ndarray:
    q = np.ascontiguousarray(q, np.int8)
    s = _f32(s)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float32)
    _check(lib().oq_sym_dequantize(_p(q), _p(s), rows, cols, group, _p(out)), "sym_dequantize")
    return out


# --------------------------------------------------------------------------
# Matmul references.
# --------------------------------------------------------------------------
def matmul_nt_f64(a, b, parallel: bool = False) -> np.ndarray:
    """C = A B^T summed in fp64 (A [M,K], B [N,K])."""
    a = _f32(a)
    b = _f32(b)
    if a.ndim == 1:
        a = a[None, :]
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    c = np.empty((m, n), np.float64)
    _check(lib(parallel).oq_matmul_nt_f64(_p(a), _p(b), m, n, k, _p(c)), "matmul_nt_f64")
    return c


def w4a16_reference(x, q, s, z, group: int = 128, parallel: bool = False) -> np.ndarray:
    """y[b, n] = sum_k x[b, k] * w_hat[n, k] with w_hat = (q - z) s, summed in fp64.
    parallel=True runs the OpenMP build (same loops per output, timing only)."""
    return matmul_nt_f64(x, asym_dequantize(q, s, z, group, parallel), parallel)


def threads(parallel: bool = True) -> int:
    """Threads the row loops of the given build use."""
    return int(lib(parallel).oq_threads())


def w8a16_reference(x, qw, b) -> np.ndarray:
    """Weight-only INT8 ("How quantization works", "Mainstream schemes at a
    glance", W8A16 row): y[t, n] = sum_k x[t, k] * (qW[n, k] * b[n]), summed in
    fp64 as b[n] * sum_k x[t, k] qW[n, k] (the integers are exact in fp32)."""
    qw = np.ascontiguousarray(qw, np.int8).astype(np.float32)
    b = _f32(b).reshape(-1).astype(np.float64)
    return matmul_nt_f64(x, qw) * b[None, :]


def int8_matmul_nt(qa, qb) -> np.ndarray:
    qa = np.ascontiguousarray(qa, np.int8)
    qb = np.ascontiguousarray(qb, np.int8)
    m, k = qa.shape
    n, k2 = qb.shape
    assert k == k2
    acc = np.empty((m, n), np.int32)
    _check(lib().oq_int8_matmul_nt(_p(qa), _p(qb), m, n, k, _p(acc)), "int8_matmul_nt (int32 overflow?)")
    return acc


def rescale_f64(acc, a, b) -> np.ndarray:
    acc = np.ascontiguousarray(acc, np.int32)
    a = _f32(a).reshape(-1)
    b = _f32(b).reshape(-1)
    m, n = acc.shape
    y = np.empty((m, n), np.float64)
    _check(lib().oq_rescale_f64(_p(acc), _p(a), _p(b), m, n, _p(y)), "rescale_f64")
    return y


# --------------------------------------------------------------------------
# SmoothQuant ("How quantization works", "Activation quantization and
# outliers"; "Quantization" (Engine Room), smoothing equation).
# --------------------------------------------------------------------------
def col_absmax(a) -> np.ndarray:
    a = _f32(a)
    rows, cols = a.shape
    out = np.empty(cols, np.float32)
    _check(lib().oq_col_absmax(_p(a), rows, cols, _p(out)), "col_absmax")
    return out


def smooth_factors(cx, cw, alpha: float = 0.5) -> np.ndarray:
    cx = _f32(cx)
    cw = _f32(cw)
    s = np.empty(cx.size, np.float32)
    _check(lib().oq_smooth_factors(_p(cx), _p(cw), cx.size, ctypes.c_float(alpha), _p(s)), "smooth_factors")
    return s


def scale_columns_mul(a, s) -> np.ndarray:
    a = _f32(a)
    s = _f32(s)
    out = np.empty_like(a)
    _check(lib().oq_scale_columns_mul(_p(a), _p(s), a.shape[0], a.shape[1], _p(out)), "scale_columns_mul")
    return out


def scale_columns_div(a, s) -> np.ndarray:
    a = _f32(a)
    s = _f32(s)
    out = np.empty_like(a)
    _check(lib().oq_scale_columns_div(_p(a), _p(s), a.shape[0], a.shape[1], _p(out)), "scale_columns_div")
    return out


def sq_quantize_weight(w, s) -> Tuple[np.ndarray, np.ndarray]:
    """Ws = W * s (columns); per-output-channel symmetric INT8 -> (qW int8 [N,K], b f32 [N])."""
    ws = scale_columns_mul(w, s) if s is not None else _f32(w)
    q, b = sym_quantize(ws, ws.shape[1], 8, 1e-8)
    return q, b.reshape(-1)


def sq_quantize_activation(x, s) -> Tuple[np.ndarray, np.ndarray]:
    """Xs = X / s (columns); per-token symmetric INT8 -> (qX int8 [M,K], a f32 [M])."""
    xs = scale_columns_div(x, s) if s is not None else _f32(x)
    q, a = sym_quantize(xs, xs.shape[1], 8, 1e-8)
    return q, a.reshape(-1)


def sq_quantize_activation_per_tensor(x, s) -> Tuple[np.ndarray, np.ndarray]:
    """Xs = X / s (columns); one symmetric INT8 scale for the whole tensor
    ("How quantization works", "Activation quantization and outliers", per-tensor
    form) -> (qX int8 [M,K], a f32 [M], every entry the tensor's scale)."""
    xs = scale_columns_div(x, s) if s is not None else _f32(x)
    q, a = sym_quantize(xs.reshape(1, -1), xs.size, 8, 1e-8)
    return q.reshape(xs.shape), np.full(xs.shape[0], a.reshape(-1)[0], np.float32)


def sq_w8a8_reference(x, s, qw, b):
    """Online W8A8 step: quantize X per token, exact int32 product, rescale.
    Returns (qX, a, acc int32, y fp64)."""
    qx, a = sq_quantize_activation(x, s)
    acc = int8_matmul_nt(qx, qw)
    return qx, a, acc, rescale_f64(acc, a, b)


# --------------------------------------------------------------------------
# FP8 E4M3 W8A8 ("How quantization works", the fake-quantization listing and
# "Mainstream schemes at a glance", FP8 row; "Quantization: Smaller Weights,
# Same Answers (Mostly)", "What about FP8, MXFP4, NVFP4 and GGUF?").
# --------------------------------------------------------------------------
def to_e4m3(a) -> np.ndarray:
    """E4M3FN code bytes of float32 values (nearest even, saturating at 448)."""
    a = _f32(a)
    out = np.empty(a.shape, np.uint8)
    _check(lib().oq_e4m3_array(_p(a), a.size, _p(out)), "to_e4m3")
    return out


def from_e4m3(b) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    _check(lib().oq_e4m3_decode_array(_p(b), b.size, _p(out)), "from_e4m3")
    return out


def fp8_quantize(x, per_tensor: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """s = max|x| / 448 per row (or one for the whole tensor), q = E4M3(x / s):
    (codes uint8 [rows, cols], scales f32 [rows], every entry the tensor's
    scale when per_tensor)."""
    x = _f32(x)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    if per_tensor:
        s = np.empty(1, np.float32)
        _check(lib().oq_fp8_quantize(_p(x), 1, x.size, x.size, _p(q), _p(s)), "fp8_quantize")
        return q, np.full(rows, s[0], np.float32)
    s = np.empty(rows, np.float32)
    _check(lib().oq_fp8_quantize(_p(x), rows, cols, cols, _p(q), _p(s)), "fp8_quantize")
    return q, s


def fp8_matmul_nt(qa, qb, parallel: bool = False) -> np.ndarray:
    """acc = decoded(qa) decoded(qb)^T summed in fp64."""
    qa = np.ascontiguousarray(qa, np.uint8)
    qb = np.ascontiguousarray(qb, np.uint8)
    m, k = qa.shape
    n, k2 = qb.shape
    assert k == k2
    acc = np.empty((m, n), np.float64)
    _check(lib(parallel).oq_fp8_matmul_nt(_p(qa), _p(qb), m, n, k, _p(acc)), "fp8_matmul_nt")
    return acc


def fp8_w8a8_reference(x, qw, b, parallel: bool = False):
    """Online FP8 W8A8: per-token E4M3 activations, exact product, rescale.
    Returns (qX, a, y fp64)."""
    qx, a = fp8_quantize(x)
    acc = fp8_matmul_nt(qx, qw, parallel)
    return qx, a, acc * a.astype(np.float64)[:, None] * np.asarray(b, np.float32).astype(np.float64)[None, :]


# --------------------------------------------------------------------------
# LLM.int8() ("Quantization" (Engine Room ch. 15), "The Mathematics": the
# vector-wise product with the outlier dimensions multiplied in 16-bit;
# "Quantization: Smaller Weights, Same Answers (Mostly)", outlier family 1).
# --------------------------------------------------------------------------
def llm_int8_reference(x, qw, b, threshold: float, max_outliers=None, x_dtype: str = "bf16"):
    """Mixed-precision decomposition of X W^T with per-output-channel INT8
    weights (qw [N, K], b [N]) and 16-bit activations x [M, K] (as float32
    values of `x_dtype`, "bf16" or "f16").  The first `max_outliers` columns
    (in column order) whose largest |x| over the batch reaches `threshold`
    are multiplied in 16-bit; the rest go through per-token INT8.
    Returns (outlier columns int32 [kept], found, qX int8 [M, K], a f32 [M],
    y fp64 [M, N])."""
    x = _f32(x)
    qw = np.ascontiguousarray(qw, np.int8)
    b = _f32(b).reshape(-1)
    m, k = x.shape
    n, k2 = qw.shape
    assert k == k2 and b.shape == (n,) and x_dtype in ("bf16", "f16")
    cap = k if max_outliers is None else int(max_outliers)
    idx = np.zeros(max(cap, 1), np.int32)
    counts = np.zeros(2, np.int64)
    qx = np.empty((m, k), np.int8)
    a = np.empty(m, np.float32)
    y = np.empty((m, n), np.float64)
    _check(lib().oq_llm_int8(_p(x), m, k, _p(qw), _p(b), n, float(threshold), cap, int(x_dtype == "bf16"),
                             _p(idx), _p(counts), _p(qx), _p(a), _p(y)), "llm_int8")
    return idx[:counts[0]].copy(), int(counts[1]), qx, a, y


AWQ_ALPHAS = np.linspace(0.0, 1.0, 11)   # the [QS] awq listing's grid, its values to the last bit


def awq_search_reference(w, x, alphas=None, parallel: bool = False, x_dtype: str = "bf16"):
    """AWQ's scaling search for weights w [N, K] and calibration activations
    x [T, K] (the 16-bit values as float32; x_dtype, "bf16" or "f16", is the
    type X / s is rounded to), INT4 groups of 128 (readings R32, R33).  Returns (err fp64 [len(alphas)], best index, s_best f32 [K], the
    codes q uint8 [N, K], scales f32 [N, K/128] and zeros uint8 [N, K/128] of
    W diag(s_best)).  parallel=True runs the OpenMP build (the same loops per
    output, the products' rows split over threads)."""
    w = _f32(w)
    x = _f32(x)
    n, k = w.shape
    t, k2 = x.shape
    assert k == k2 and k % 128 == 0
    assert x_dtype in ("bf16", "f16")
    a = np.ascontiguousarray(AWQ_ALPHAS if alphas is None else alphas, np.float64).reshape(-1)
    err = np.empty(a.size, np.float64)
    best = np.zeros(1, np.int64)
    s = np.empty(k, np.float32)
    q = np.empty((n, k), np.uint8)
    sc = np.empty((n, k // 128), np.float32)
    z = np.empty((n, k // 128), np.uint8)
    _check(lib(parallel).oq_awq_search(_p(w), _p(x), n, k, t, _p(a), a.size, _p(err), _p(best), _p(s), _p(q), _p(sc),
                                       _p(z), 1 if x_dtype == "f16" else 0), "awq_search")
    return err, int(best[0]), s, q, sc, z


def awq_factors_reference(x, alphas=None):
    """AWQ's factors s [len(alphas), K] for calibration activations x [T, K] (R33)."""
    x = _f32(x)
    t, k = x.shape
    a = np.ascontiguousarray(AWQ_ALPHAS if alphas is None else alphas, np.float64).reshape(-1)
    s = np.empty((a.size, k), np.float32)
    _check(lib().oq_awq_factors(_p(x), k, t, _p(a), a.size, _p(s)), "awq_factors")
    return s
