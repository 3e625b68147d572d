"""Group-wise INT4 weight quantization and quantized matmuls for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libqmm.so`` (declared in
``include/qmm.h``).  It only marshals arguments: it allocates output tensors
with torch (device memory), passes raw device pointers and the current HIP
stream, and turns a non-zero status into ``QmmError``.  Every computation runs
in the library's hand-written HIP kernels; there is no fallback path, and the
functions raise if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "QmmError", "lib", "library_path", "F32", "F16", "BF16", "I32", "GROUP",
    "w4_sizes", "quantize_groupwise", "quantize_groupwise_symmetric", "dequantize", "w4a16_gemv", "w4a16_gemm",
    "w8a16_gemv",
    "sq_smooth_factors", "sq_quantize_weight", "sq_quantize_activation", "sq_quantize_activation_per_tensor",
    "sq_int8_gemm",
    "sq_workspace_bytes", "smooth_quant_w8a8_gemm", "smooth_quant_w8a8_gemm_noalloc", "SQ_STATIC_SCRATCH_BYTES",
]

F32, F16, BF16, I32 = 0, 1, 2, 3
GROUP = 128
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int32: I32}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libqmm.so")


class QmmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().qmm_status_string(status).decode() if status else "ok"
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

# name -> argument types of the C ABI
_P, _I64, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "qmm_status_string": ([_I], ctypes.c_char_p),
    "qmm_version": ([], _I),
    "qmm_w4_sizes": ([_I64, _I64, _I, _P, _P, _P], _I),
    "quantize_groupwise": ([_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P], _I),
    "quantize_groupwise_symmetric": ([_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P], _I),
    "dequantize": ([_P, _P, _P, _I64, _I64, _I, _I, _P, _I, _P], _I),
    "w4a16_gemv": ([_P, _P, _P, _I64, _I64, _I, _P, _I, _I64, _P, _I, _P], _I),
    "w4a16_gemm": ([_P, _P, _P, _I64, _I64, _I, _P, _I, _I64, _P, _I, _P], _I),
    "w8a16_gemv": ([_P, _P, _I64, _I64, _P, _I, _I64, _P, _I, _P], _I),
    "sq_smooth_factors": ([_P, _I, _I64, _P, _I, _I64, _I64, _F, _P, _P, _P, _P], _I),
    "sq_quantize_weight": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_quantize_activation": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_quantize_activation_per_tensor": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_int8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "sq_workspace_bytes": ([_I64, _I64], _SZ),
    "smooth_quant_w8a8_gemm": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P], _I),
    "smooth_quant_w8a8_gemm_noalloc": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
}

# Device scratch of smooth_quant_w8a8_gemm_noalloc (QMM_SQ_STATIC_SCRATCH_BYTES).
SQ_STATIC_SCRATCH_BYTES = 16 * 1024 * 1024 + 64 * 1024


def lib() -> ctypes.CDLL:
    """The loaded libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with __graft_entry__.build() "
                              "(python -m quantized_matmul_quantize_amd._build)")
        l = ctypes.CDLL(library_path)
        for name, (argtypes, restype) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = l
    return _lib


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise QmmError(name, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dt(dtype: torch.dtype) -> int:
    if dtype not in _DT:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DT[dtype]


def w4_sizes(N: int, K: int, group: int = GROUP) -> Tuple[int, int, int]:
    """(codes, scales, zeros) byte sizes of the INT4 format."""
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _call("qmm_w4_sizes", N, K, group, ctypes.byref(c), ctypes.byref(s), ctypes.byref(z))
    return c.value, s.value, z.value


def quantize_groupwise(W: torch.Tensor, group: int = GROUP, bits: int = 4, symmetric: bool = False):
    """W [N, K] (fp32 / bf16 / fp16) -> codes u8 [N, K/2], scales f32 [N, G], zeros u8 [N, ceil(G/2)].
    symmetric=True: the symmetric grid, stored with zero-point 8 in the same format."""
    _check(W, "W")
    N, K = W.shape
    G = K // group if group > 0 else 0
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, max(G, 1)), dtype=torch.float32, device=W.device)
    zeros = torch.empty((N, max((G + 1) // 2, 1)), dtype=torch.uint8, device=W.device)
    _call("quantize_groupwise_symmetric" if symmetric else "quantize_groupwise", _ptr(W), _dt(W.dtype), N, K, group,
          bits, _ptr(codes), _ptr(scales), _ptr(zeros), _stream(W))
    return codes, scales, zeros


def quantize_groupwise_symmetric(W: torch.Tensor, group: int = GROUP, bits: int = 4):
    """Symmetric per-group INT4 in the asymmetric storage format (zero-point 8)."""
    return quantize_groupwise(W, group, bits, symmetric=True)


def dequantize(codes, scales, zeros, dtype: torch.dtype = torch.float32, group: int = GROUP, bits: int = 4):
    """INT4 format -> W_hat [N, K] in dtype."""
    _check(codes, "codes")
    N, K = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((N, K), dtype=dtype, device=codes.device)
    _call("dequantize", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, bits, _ptr(out), _dt(dtype),
          _stream(codes))
    return out


def w4a16_gemv(codes, scales, zeros, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, out: Optional[torch.Tensor] = None):
    """y [B, N] = x [B, K] @ W_hat^T for B <= 8 (decode)."""
    _check(codes, "codes")
    _check(x, "x")
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    N, K = codes.shape[0], codes.shape[1] * 2
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, N), dtype=out_dtype or x.dtype, device=x.device)
    _call("w4a16_gemv", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, _ptr(x2), _dt(x2.dtype), B, _ptr(out),
          _dt(out.dtype), _stream(x))
    return out


def w4a16_gemm(codes, scales, zeros, X: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, out: Optional[torch.Tensor] = None):
    """Y [M, N] = X [M, K] @ W_hat^T (bf16 or fp16 activations, fp32 accumulation)."""
    _check(codes, "codes")
    _check(X, "X")
    N, K = codes.shape[0], codes.shape[1] * 2
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or X.dtype, device=X.device)
    _call("w4a16_gemm", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, _ptr(X), _dt(X.dtype), M, _ptr(out),
          _dt(out.dtype), _stream(X))
    return out


def w8a16_gemv(qW, w_scale, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               out: Optional[torch.Tensor] = None):
    """y [B, N] = w_scale[n] * (x [B, K] @ qW^T) for B <= 8 (weight-only INT8 decode)."""
    _check(qW, "qW")
    _check(x, "x")
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    N, K = qW.shape
    B = x2.shape[0]
    if out is None:
        out = torch.empty((B, N), dtype=out_dtype or x.dtype, device=x.device)
    _call("w8a16_gemv", _ptr(qW), _ptr(w_scale), N, K, _ptr(x2), _dt(x2.dtype), B, _ptr(out), _dt(out.dtype),
          _stream(x))
    return out


def sq_smooth_factors(X: torch.Tensor, W: torch.Tensor, alpha: float = 0.5):
    """-> (smooth [K], x_colmax [K], w_colmax [K]) float32."""
    _check(X, "X")
    _check(W, "W")
    M, K = X.shape
    N = W.shape[0]
    smooth = torch.empty(K, dtype=torch.float32, device=X.device)
    cx = torch.empty_like(smooth)
    cw = torch.empty_like(smooth)
    _call("sq_smooth_factors", _ptr(X), _dt(X.dtype), M, _ptr(W), _dt(W.dtype), N, K, alpha, _ptr(cx), _ptr(cw),
          _ptr(smooth), _stream(X))
    return smooth, cx, cw


def sq_quantize_weight(W: torch.Tensor, smooth: Optional[torch.Tensor] = None):
    """-> (qW int8 [N, K], w_scale f32 [N])."""
    _check(W, "W")
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    s = torch.empty(N, dtype=torch.float32, device=W.device)
    _call("sq_quantize_weight", _ptr(W), _dt(W.dtype), _ptr(smooth), N, K, _ptr(q), _ptr(s), _stream(W))
    return q, s


def sq_quantize_activation(X: torch.Tensor, smooth: Optional[torch.Tensor] = None, per_tensor: bool = False):
    """-> (qX int8 [M, K], x_scale f32 [M]); per_tensor=True: one scale for the whole X, repeated per row."""
    _check(X, "X")
    M, K = X.shape
    q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    s = torch.empty(M, dtype=torch.float32, device=X.device)
    _call("sq_quantize_activation_per_tensor" if per_tensor else "sq_quantize_activation", _ptr(X), _dt(X.dtype),
          _ptr(smooth), M, K, _ptr(q), _ptr(s), _stream(X))
    return q, s


def sq_quantize_activation_per_tensor(X: torch.Tensor, smooth: Optional[torch.Tensor] = None):
    """-> (qX int8 [M, K], x_scale f32 [M]) with one scale for the whole X, repeated per row."""
    return sq_quantize_activation(X, smooth, per_tensor=True)


def sq_int8_gemm(qX, x_scale, qW, w_scale, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None):
    """Y [M, N] = (qX qW^T) * x_scale[m] * w_scale[n]; out_dtype int32 returns the raw accumulator."""
    _check(qX, "qX")
    _check(qW, "qW")
    M, K = qX.shape
    N = qW.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qX.device)
    _call("sq_int8_gemm", _ptr(qX), _ptr(x_scale), _ptr(qW), _ptr(w_scale), M, N, K, _ptr(out), _dt(out.dtype),
          _stream(qX))
    return out


def sq_workspace_bytes(M: int, K: int) -> int:
    return int(lib().sq_workspace_bytes(M, K))


def smooth_quant_w8a8_gemm(X: torch.Tensor, smooth: Optional[torch.Tensor], qW, w_scale,
                           out_dtype: torch.dtype = torch.bfloat16, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None):
    """Online W8A8 step: per-token smoothing + INT8 quantization of X, INT8 GEMM, rescale."""
    _check(X, "X")
    M, K = X.shape
    N = qW.shape[0]
    need = sq_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _call("smooth_quant_w8a8_gemm", _ptr(X), _dt(X.dtype), _ptr(smooth), _ptr(qW), _ptr(w_scale), M, N, K,
          _ptr(out), _dt(out.dtype), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(X))
    return out


def smooth_quant_w8a8_gemm_noalloc(X: torch.Tensor, smooth: Optional[torch.Tensor], qW, w_scale,
                                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """smooth_quant_w8a8_gemm with the library's own device scratch instead of a
    workspace (for callers that cannot allocate; pass `out` to allocate nothing)."""
    _check(X, "X")
    M, K = X.shape
    N = qW.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _call("smooth_quant_w8a8_gemm_noalloc", _ptr(X), _dt(X.dtype), _ptr(smooth), _ptr(qW), _ptr(w_scale), M, N, K,
          _ptr(out), _dt(out.dtype), _stream(X))
    return out
