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

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
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
        }
        for name, argtypes in sigs.items():
            fn = getattr(_lib, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
    return _lib


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


def asym_dequantize(q, s, z, group: int = 128) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s = _f32(s)
    z = np.ascontiguousarray(z, np.uint8)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float32)
    _check(lib().oq_asym_dequantize(_p(q), _p(s), _p(z), rows, cols, group, _p(out)), "asym_dequantize")
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
def matmul_nt_f64(a, b) -> np.ndarray:
    """C = A B^T summed in fp64 (A [M,K], B [N,K])."""
    a = _f32(a)
    b = _f32(b)
    if a.ndim == 1:
        a = a[None, :]
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    c = np.empty((m, n), np.float64)
    _check(lib().oq_matmul_nt_f64(_p(a), _p(b), m, n, k, _p(c)), "matmul_nt_f64")
    return c


def w4a16_reference(x, q, s, z, group: int = 128) -> np.ndarray:
    """y[b, n] = sum_k x[b, k] * w_hat[n, k] with w_hat = (q - z) s, summed in fp64."""
    return matmul_nt_f64(x, asym_dequantize(q, s, z, group))


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
