"""Group-wise INT4 weight quantization and quantized matmuls for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libqmm.so`` (declared in
``include/qmm.h``).  It only marshals arguments: it checks every tensor's
shape, dtype, device and layout against the call (``ValueError`` before any
launch), allocates output tensors with torch (device memory), passes raw
device pointers and the current HIP stream, and turns a non-zero status into
``QmmError``.  Every computation runs in the library's hand-written HIP
kernels; there is no fallback path, and the functions raise if the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "QmmError", "lib", "library_path", "F32", "F16", "BF16", "I32", "GROUP", "SQ_STATIC_SCRATCH_BYTES",
    "w4_sizes", "wq_sizes", "quantize_groupwise", "quantize_groupwise_symmetric", "quantize_groupwise_ex",
    "dequantize", "dequantize_ex", "w4a16_gemv", "w4a16_gemm", "wxa16_gemv", "wxa16_gemm",
    "w4_repack_from_plain", "w4_repack_to_plain", "w8a16_gemv",
    "sq_smooth_factors", "sq_quantize_weight", "sq_quantize_activation", "sq_quantize_activation_per_tensor",
    "sq_int8_gemm", "sq_workspace_bytes", "smooth_quant_w8a8_gemm", "smooth_quant_w8a8_gemm_noalloc",
    "fp8_quantize", "fp8_gemm", "fp8_w8a8_gemm",
    "llm_int8_outliers", "llm_int8_workspace_bytes", "llm_int8_gemm", "awq_workspace_bytes", "awq_search", "stream_read",
]

F32, F16, BF16, I32 = 0, 1, 2, 3
GROUP = 128
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int32: I32}
_FLOATS = (torch.float32, torch.bfloat16, torch.float16)
_HALVES = (torch.bfloat16, torch.float16)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libqmm.so")

# Device scratch of smooth_quant_w8a8_gemm_noalloc (QMM_SQ_STATIC_SCRATCH_BYTES).
SQ_STATIC_SCRATCH_BYTES = 16 * 1024 * 1024 + 64 * 1024


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
    "qmm_wq_sizes": ([_I64, _I64, _I, _I, _I, _P, _P, _P], _I),
    "quantize_groupwise": ([_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P], _I),
    "quantize_groupwise_symmetric": ([_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _P], _I),
    "quantize_groupwise_ex": ([_P, _I, _I64, _I64, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "dequantize": ([_P, _P, _P, _I64, _I64, _I, _I, _P, _I, _P], _I),
    "dequantize_ex": ([_P, _P, _P, _I64, _I64, _I, _I, _I, _P, _I, _P], _I),
    "w4a16_gemv": ([_P, _P, _P, _I64, _I64, _I, _P, _I, _I64, _P, _I, _P], _I),
    "w4a16_gemm": ([_P, _P, _P, _I64, _I64, _I, _P, _I, _I64, _P, _I, _P], _I),
    "wxa16_gemv": ([_P, _P, _P, _I64, _I64, _I, _I, _I, _P, _I, _I64, _P, _I, _P], _I),
    "wxa16_gemm": ([_P, _P, _P, _I64, _I64, _I, _I, _I, _P, _I, _I64, _P, _I, _P], _I),
    "qmm_w4_repack_from_plain": ([_P, _P, _I64, _I64, _P], _I),
    "qmm_w4_repack_to_plain": ([_P, _P, _I64, _I64, _P], _I),
    "w8a16_gemv": ([_P, _P, _I64, _I64, _P, _I, _I64, _P, _I, _P], _I),
    "sq_smooth_factors": ([_P, _I, _I64, _P, _I, _I64, _I64, _F, _P, _P, _P, _P], _I),
    "sq_quantize_weight": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_quantize_activation": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_quantize_activation_per_tensor": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "sq_int8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "sq_workspace_bytes": ([_I64, _I64], _SZ),
    "smooth_quant_w8a8_gemm": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P], _I),
    "smooth_quant_w8a8_gemm_noalloc": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "fp8_quantize": ([_P, _I, _I64, _I64, _I, _P, _P, _P], _I),
    "fp8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "fp8_w8a8_gemm": ([_P, _I, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P], _I),
    "llm_int8_outliers": ([_P, _I, _I64, _I64, _F, _I64, _P, _P, _P, _P], _I),
    "llm_int8_workspace_bytes": ([_I64, _I64, _I64, _I64], _SZ),
    "awq_workspace_bytes": ([_I64, _I64, _I64, _I64], _SZ),
    "qmm_stream_read": ([_P, _SZ, _P, _P], _I),
    "awq_search": ([_P, _I, _P, _I, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "llm_int8_gemm": ([_P, _I, _P, _P, _I64, _I64, _I64, _F, _I64, _P, _I, _P, _P, _SZ, _P], _I),
}


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


def _dt(dtype: torch.dtype) -> int:
    if dtype not in _DT:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DT[dtype]


def _req(t, name: str, dtypes: Sequence[torch.dtype], shape: Optional[Tuple] = None,
         ndim: Optional[int] = None) -> None:
    """Check one operand's dtype and shape (None entries are free) or number
    of dimensions.  Raises ValueError."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {list(dtypes)}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(a) != int(s) for a, s in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")


def _place(**tensors) -> torch.device:
    """After every shape and dtype check: all operands on one GPU, contiguous.
    Returns their device.  None entries (optional operands) are skipped."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return dev


def _out(out: Optional[torch.Tensor], shape: Tuple, dtype: torch.dtype, name: str = "out") -> None:
    if out is not None:
        _req(out, name, (dtype,), shape=shape)


def _alloc(out: Optional[torch.Tensor], shape: Tuple, dtype: torch.dtype, device) -> torch.Tensor:
    return out if out is not None else torch.empty(shape, dtype=dtype, device=device)


def _sdt(scale_dtype: torch.dtype) -> int:
    if scale_dtype not in (torch.float32, torch.float16):
        raise ValueError(f"scale_dtype must be torch.float32 or torch.float16, not {scale_dtype}")
    return _DT[scale_dtype]


def _groups(K: int, group: int) -> int:
    if group <= 0 or K % group:
        raise ValueError(f"K = {K} is not a multiple of the group size {group}")
    return K // group


def _code_cols(K: int, bits: int) -> int:
    return K * bits // 8


def _zero_cols(G: int, bits: int) -> int:
    return (G + 1) // 2 if bits <= 4 else G


def _k_from_codes(codes: torch.Tensor, bits: int) -> int:
    if bits not in (3, 4, 8):
        raise ValueError(f"bits must be 3, 4 or 8, not {bits}")
    if codes.dim() != 2 or (codes.shape[1] * 8) % bits:
        raise ValueError(f"codes of shape {tuple(codes.shape)} do not hold {bits}-bit codes")
    return codes.shape[1] * 8 // bits


def _check_format(codes, scales, zeros, group: int, bits: int, scale_dtype: torch.dtype):
    """Shapes and dtypes of the stored-format operands of one weight matrix; returns (N, K)."""
    if not isinstance(codes, torch.Tensor):
        raise ValueError("codes must be a torch.Tensor")
    K = _k_from_codes(codes, bits)
    N = codes.shape[0]
    G = _groups(K, group)
    _req(codes, "codes", (torch.uint8,), shape=(N, _code_cols(K, bits)))
    _req(scales, "scales", (scale_dtype,), shape=(N, G))
    _req(zeros, "zeros", (torch.uint8,), shape=(N, _zero_cols(G, bits)))
    return N, K


def _tokens(x: torch.Tensor, K: int, name: str, dtypes=_HALVES) -> torch.Tensor:
    """Activations [T, K] (a 1-D [K] vector is one token)."""
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    _req(x2, name, dtypes, shape=(None, K))
    return x2


# ---------------------------------------------------------------------------
# Sizes.
# ---------------------------------------------------------------------------
def w4_sizes(N: int, K: int, group: int = GROUP) -> Tuple[int, int, int]:
    """(codes, scales, zeros) byte sizes of the INT4 format."""
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _call("qmm_w4_sizes", N, K, group, ctypes.byref(c), ctypes.byref(s), ctypes.byref(z))
    return c.value, s.value, z.value


def wq_sizes(N: int, K: int, group: int = GROUP, bits: int = 4,
             scale_dtype: torch.dtype = torch.float32) -> Tuple[int, int, int]:
    """(codes, scales, zeros) byte sizes of any stored format."""
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _call("qmm_wq_sizes", N, K, group, bits, _sdt(scale_dtype), ctypes.byref(c), ctypes.byref(s), ctypes.byref(z))
    return c.value, s.value, z.value


# ---------------------------------------------------------------------------
# Quantization and dequantization.
# ---------------------------------------------------------------------------
def _quant_outputs(W, group, bits, scale_dtype):
    _req(W, "W", _FLOATS, ndim=2)
    if bits not in (3, 4, 8):
        raise ValueError(f"bits must be 3, 4 or 8, not {bits}")
    N, K = W.shape
    G = _groups(K, group)
    dev = _place(W=W)
    codes = torch.empty((N, _code_cols(K, bits)), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, G), dtype=scale_dtype, device=dev)
    zeros = torch.empty((N, _zero_cols(G, bits)), dtype=torch.uint8, device=dev)
    return N, K, codes, scales, zeros


def quantize_groupwise_ex(W: torch.Tensor, group: int = GROUP, bits: int = 4,
                          scale_dtype: torch.dtype = torch.float32, symmetric: bool = False):
    """W [N, K] (fp32 / bf16 / fp16) -> (codes, scales, zeros) in a stored format:
    group 32..1024, 3, 4 or 8 bits, fp32 or fp16 scales, asymmetric or symmetric grid."""
    sdt = _sdt(scale_dtype)
    N, K, codes, scales, zeros = _quant_outputs(W, group, bits, scale_dtype)
    _call("quantize_groupwise_ex", _ptr(W), _dt(W.dtype), N, K, group, bits, sdt, int(symmetric),
          _ptr(codes), _ptr(scales), _ptr(zeros), _stream(W))
    return codes, scales, zeros


def quantize_groupwise(W: torch.Tensor, group: int = GROUP, bits: int = 4, symmetric: bool = False):
    """W [N, K] (fp32 / bf16 / fp16) -> codes u8 [N, K/2], scales f32 [N, G], zeros u8 [N, ceil(G/2)]
    (other group sizes / bit widths: the stored formats with fp32 scales).
    symmetric=True: the symmetric grid, stored with zero-point 2^(bits-1) in the same format."""
    N, K, codes, scales, zeros = _quant_outputs(W, group, bits, torch.float32)
    _call("quantize_groupwise_symmetric" if symmetric else "quantize_groupwise", _ptr(W), _dt(W.dtype), N, K, group,
          bits, _ptr(codes), _ptr(scales), _ptr(zeros), _stream(W))
    return codes, scales, zeros


def quantize_groupwise_symmetric(W: torch.Tensor, group: int = GROUP, bits: int = 4):
    """Symmetric per-group quantization in the asymmetric storage format (zero-point 2^(bits-1))."""
    return quantize_groupwise(W, group, bits, symmetric=True)


def _scale_dtype_of(scales) -> torch.dtype:
    if not isinstance(scales, torch.Tensor):
        raise ValueError("scales must be a torch.Tensor")
    _sdt(scales.dtype)
    return scales.dtype


def dequantize_ex(codes, scales, zeros, dtype: torch.dtype = torch.float32, group: int = GROUP, bits: int = 4,
                  out: Optional[torch.Tensor] = None):
    """Stored format -> W_hat [N, K] in dtype (the scales' dtype selects fp32 or fp16 scales)."""
    sdt = _scale_dtype_of(scales)
    N, K = _check_format(codes, scales, zeros, group, bits, sdt)
    if dtype not in _FLOATS:
        raise ValueError(f"unsupported output dtype {dtype}")
    _out(out, (N, K), dtype)
    dev = _place(codes=codes, scales=scales, zeros=zeros, out=out)
    out = _alloc(out, (N, K), dtype, dev)
    _call("dequantize_ex", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, bits, _sdt(sdt), _ptr(out), _dt(dtype),
          _stream(codes))
    return out


def dequantize(codes, scales, zeros, dtype: torch.dtype = torch.float32, group: int = GROUP, bits: int = 4,
               out: Optional[torch.Tensor] = None):
    """Stored format with fp32 scales -> W_hat [N, K] in dtype."""
    N, K = _check_format(codes, scales, zeros, group, bits, torch.float32)
    if dtype not in _FLOATS:
        raise ValueError(f"unsupported output dtype {dtype}")
    _out(out, (N, K), dtype)
    dev = _place(codes=codes, scales=scales, zeros=zeros, out=out)
    out = _alloc(out, (N, K), dtype, dev)
    _call("dequantize", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, bits, _ptr(out), _dt(dtype),
          _stream(codes))
    return out


# ---------------------------------------------------------------------------
# Weight-only matmuls.
# ---------------------------------------------------------------------------
def _mm_args(codes, scales, zeros, x, group, bits, sdt, out, out_dtype, max_tokens=None, name="x"):
    N, K = _check_format(codes, scales, zeros, group, bits, sdt)
    x2 = _tokens(x, K, name)
    T = x2.shape[0]
    if max_tokens is not None and not 1 <= T <= max_tokens:
        raise ValueError(f"takes 1 to {max_tokens} tokens, not {T}")
    odt = out.dtype if out is not None else (out_dtype or x2.dtype)
    _out(out, (T, N), odt)
    dev = _place(codes=codes, scales=scales, zeros=zeros, **{name: x2}, out=out)
    return N, K, T, x2, _alloc(out, (T, N), odt, dev)


def w4a16_gemv(codes, scales, zeros, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, out: Optional[torch.Tensor] = None):
    """y [B, N] = x [B, K] @ W_hat^T for B <= 8 (decode), INT4 codes with fp32 scales."""
    N, K, B, x2, out = _mm_args(codes, scales, zeros, x, group, 4, torch.float32, out, out_dtype, 8)
    _call("w4a16_gemv", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, _ptr(x2), _dt(x2.dtype), B, _ptr(out),
          _dt(out.dtype), _stream(x2))
    return out


def w4a16_gemm(codes, scales, zeros, X: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, out: Optional[torch.Tensor] = None):
    """Y [M, N] = X [M, K] @ W_hat^T (bf16 or fp16 activations, fp32 accumulation)."""
    N, K, M, X2, out = _mm_args(codes, scales, zeros, X, group, 4, torch.float32, out, out_dtype, None, "X")
    _call("w4a16_gemm", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, _ptr(X2), _dt(X2.dtype), M, _ptr(out),
          _dt(out.dtype), _stream(X2))
    return out


def wxa16_gemv(codes, scales, zeros, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, bits: int = 4, out: Optional[torch.Tensor] = None):
    """y [B, N] = x [B, K] @ W_hat^T for B <= 8 on any stored format (the scales' dtype selects fp32 / fp16)."""
    sdt = _scale_dtype_of(scales)
    N, K, B, x2, out = _mm_args(codes, scales, zeros, x, group, bits, sdt, out, out_dtype, 8)
    _call("wxa16_gemv", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, bits, _sdt(sdt), _ptr(x2), _dt(x2.dtype),
          B, _ptr(out), _dt(out.dtype), _stream(x2))
    return out


def wxa16_gemm(codes, scales, zeros, X: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               group: int = GROUP, bits: int = 4, out: Optional[torch.Tensor] = None):
    """Y [M, N] = X [M, K] @ W_hat^T on any stored format."""
    sdt = _scale_dtype_of(scales)
    N, K, M, X2, out = _mm_args(codes, scales, zeros, X, group, bits, sdt, out, out_dtype, None, "X")
    _call("wxa16_gemm", _ptr(codes), _ptr(scales), _ptr(zeros), N, K, group, bits, _sdt(sdt), _ptr(X2), _dt(X2.dtype),
          M, _ptr(out), _dt(out.dtype), _stream(X2))
    return out


def _repack(name, src, out, what):
    _req(src, what, (torch.uint8,), ndim=2)
    _out(out, tuple(src.shape), torch.uint8)
    dev = _place(**{what: src}, out=out)
    out = _alloc(out, tuple(src.shape), torch.uint8, dev)
    _call(name, _ptr(src), _ptr(out), src.shape[0], src.shape[1] * 2, _stream(src))
    return out


def w4_repack_from_plain(plain: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """4-bit codes [N, K/2] in plain nibble order -> the library's code words (same shape)."""
    return _repack("qmm_w4_repack_from_plain", plain, out, "plain")


def w4_repack_to_plain(codes: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The library's 4-bit code words [N, K/2] -> plain nibble order (same shape)."""
    return _repack("qmm_w4_repack_to_plain", codes, out, "codes")


def w8a16_gemv(qW, w_scale, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
               out: Optional[torch.Tensor] = None):
    """y [B, N] = w_scale[n] * (x [B, K] @ qW^T) for B <= 8 (weight-only INT8 decode)."""
    _req(qW, "qW", (torch.int8,), ndim=2)
    N, K = qW.shape
    _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    x2 = _tokens(x, K, "x")
    B = x2.shape[0]
    if not 1 <= B <= 8:
        raise ValueError(f"w8a16_gemv takes 1 to 8 tokens, not {B}")
    odt = out.dtype if out is not None else (out_dtype or x2.dtype)
    _out(out, (B, N), odt)
    dev = _place(qW=qW, w_scale=w_scale, x=x2, out=out)
    out = _alloc(out, (B, N), odt, dev)
    _call("w8a16_gemv", _ptr(qW), _ptr(w_scale), N, K, _ptr(x2), _dt(x2.dtype), B, _ptr(out), _dt(out.dtype),
          _stream(x2))
    return out


# ---------------------------------------------------------------------------
# SmoothQuant W8A8.
# ---------------------------------------------------------------------------
def _smooth_arg(smooth, K: int) -> None:
    if smooth is not None:
        _req(smooth, "smooth", (torch.float32,), shape=(K,))


def sq_smooth_factors(X: torch.Tensor, W: torch.Tensor, alpha: float = 0.5):
    """-> (smooth [K], x_colmax [K], w_colmax [K]) float32."""
    _req(X, "X", _FLOATS, ndim=2)
    M, K = X.shape
    _req(W, "W", _FLOATS, shape=(None, K))
    N = W.shape[0]
    dev = _place(X=X, W=W)
    smooth = torch.empty(K, dtype=torch.float32, device=dev)
    cx = torch.empty_like(smooth)
    cw = torch.empty_like(smooth)
    _call("sq_smooth_factors", _ptr(X), _dt(X.dtype), M, _ptr(W), _dt(W.dtype), N, K, alpha, _ptr(cx), _ptr(cw),
          _ptr(smooth), _stream(X))
    return smooth, cx, cw


def sq_quantize_weight(W: torch.Tensor, smooth: Optional[torch.Tensor] = None):
    """-> (qW int8 [N, K], w_scale f32 [N])."""
    _req(W, "W", _FLOATS, ndim=2)
    N, K = W.shape
    _smooth_arg(smooth, K)
    dev = _place(W=W, smooth=smooth)
    q = torch.empty((N, K), dtype=torch.int8, device=dev)
    s = torch.empty(N, dtype=torch.float32, device=dev)
    _call("sq_quantize_weight", _ptr(W), _dt(W.dtype), _ptr(smooth), N, K, _ptr(q), _ptr(s), _stream(W))
    return q, s


def sq_quantize_activation(X: torch.Tensor, smooth: Optional[torch.Tensor] = None, per_tensor: bool = False):
    """-> (qX int8 [M, K], x_scale f32 [M]); per_tensor=True: one scale for the whole X, repeated per row."""
    _req(X, "X", _FLOATS, ndim=2)
    M, K = X.shape
    _smooth_arg(smooth, K)
    dev = _place(X=X, smooth=smooth)
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    _call("sq_quantize_activation_per_tensor" if per_tensor else "sq_quantize_activation", _ptr(X), _dt(X.dtype),
          _ptr(smooth), M, K, _ptr(q), _ptr(s), _stream(X))
    return q, s


def sq_quantize_activation_per_tensor(X: torch.Tensor, smooth: Optional[torch.Tensor] = None):
    """-> (qX int8 [M, K], x_scale f32 [M]) with one scale for the whole X, repeated per row."""
    return sq_quantize_activation(X, smooth, per_tensor=True)


def sq_int8_gemm(qX, x_scale, qW, w_scale, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None):
    """Y [M, N] = (qX qW^T) * x_scale[m] * w_scale[n]; out_dtype int32 returns the raw accumulator."""
    _req(qX, "qX", (torch.int8,), ndim=2)
    M, K = qX.shape
    _req(qW, "qW", (torch.int8,), shape=(None, K))
    N = qW.shape[0]
    odt = out.dtype if out is not None else out_dtype
    raw = odt == torch.int32
    if not raw:
        _req(x_scale, "x_scale", (torch.float32,), shape=(M,))
        _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    _out(out, (M, N), odt)
    dev = _place(qX=qX, qW=qW, x_scale=None if raw else x_scale, w_scale=None if raw else w_scale, out=out)
    out = _alloc(out, (M, N), odt, dev)
    _call("sq_int8_gemm", _ptr(qX), _ptr(x_scale), _ptr(qW), _ptr(w_scale), M, N, K, _ptr(out), _dt(out.dtype),
          _stream(qX))
    return out


def sq_workspace_bytes(M: int, K: int) -> int:
    return int(lib().sq_workspace_bytes(M, K))


def _online_args(X, smooth, qW, w_scale, out, out_dtype, workspace=None):
    _req(X, "X", _FLOATS, ndim=2)
    M, K = X.shape
    _smooth_arg(smooth, K)
    _req(qW, "qW", (torch.int8,), shape=(None, K))
    N = qW.shape[0]
    _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    odt = out.dtype if out is not None else out_dtype
    _out(out, (M, N), odt)
    if workspace is not None:
        _req(workspace, "workspace", (torch.uint8,), ndim=1)
        if workspace.numel() < sq_workspace_bytes(M, K):
            raise ValueError(f"workspace holds {workspace.numel()} bytes; {sq_workspace_bytes(M, K)} needed")
    dev = _place(X=X, smooth=smooth, qW=qW, w_scale=w_scale, out=out, workspace=workspace)
    return M, N, K, dev, _alloc(out, (M, N), odt, dev)


def smooth_quant_w8a8_gemm(X: torch.Tensor, smooth: Optional[torch.Tensor], qW, w_scale,
                           out_dtype: torch.dtype = torch.bfloat16, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None):
    """Online W8A8 step: per-token smoothing + INT8 quantization of X, INT8 GEMM, rescale."""
    M, N, K, dev, out = _online_args(X, smooth, qW, w_scale, out, out_dtype, workspace)
    if workspace is None:
        workspace = torch.empty(sq_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    _call("smooth_quant_w8a8_gemm", _ptr(X), _dt(X.dtype), _ptr(smooth), _ptr(qW), _ptr(w_scale), M, N, K,
          _ptr(out), _dt(out.dtype), _ptr(workspace), workspace.numel(), _stream(X))
    return out


def smooth_quant_w8a8_gemm_noalloc(X: torch.Tensor, smooth: Optional[torch.Tensor], qW, w_scale,
                                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """smooth_quant_w8a8_gemm with the library's own device scratch instead of a
    workspace (for callers that cannot allocate; pass `out` to allocate nothing)."""
    M, N, K, dev, out = _online_args(X, smooth, qW, w_scale, out, out_dtype)
    _call("smooth_quant_w8a8_gemm_noalloc", _ptr(X), _dt(X.dtype), _ptr(smooth), _ptr(qW), _ptr(w_scale), M, N, K,
          _ptr(out), _dt(out.dtype), _stream(X))
    return out


# ---------------------------------------------------------------------------
# FP8 E4M3 W8A8 (codes are torch.uint8 holding OCP E4M3 bytes; view them as
# torch.float8_e4m3fn to read the values).
# ---------------------------------------------------------------------------
def fp8_quantize(X: torch.Tensor, per_tensor: bool = False):
    """-> (q uint8 [rows, K] E4M3 codes, scale f32 [rows]); s = max|x| / 448 per
    row, or one for the whole matrix (repeated per row) when per_tensor."""
    _req(X, "X", _FLOATS, ndim=2)
    rows, K = X.shape
    dev = _place(X=X)
    q = torch.empty((rows, K), dtype=torch.uint8, device=dev)
    s = torch.empty(rows, dtype=torch.float32, device=dev)
    _call("fp8_quantize", _ptr(X), _dt(X.dtype), rows, K, int(per_tensor), _ptr(q), _ptr(s), _stream(X))
    return q, s


def fp8_gemm(qX, x_scale, qW, w_scale, out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Y [M, N] = (E4M3(qX) E4M3(qW)^T) * x_scale[m] * w_scale[n] (fp32 accumulation)."""
    _req(qX, "qX", (torch.uint8,), ndim=2)
    M, K = qX.shape
    _req(qW, "qW", (torch.uint8,), shape=(None, K))
    N = qW.shape[0]
    _req(x_scale, "x_scale", (torch.float32,), shape=(M,))
    _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    odt = out.dtype if out is not None else out_dtype
    _out(out, (M, N), odt)
    dev = _place(qX=qX, qW=qW, x_scale=x_scale, w_scale=w_scale, out=out)
    out = _alloc(out, (M, N), odt, dev)
    _call("fp8_gemm", _ptr(qX), _ptr(x_scale), _ptr(qW), _ptr(w_scale), M, N, K, _ptr(out), _dt(out.dtype),
          _stream(qX))
    return out


def fp8_w8a8_gemm(X: torch.Tensor, qW, w_scale, out_dtype: torch.dtype = torch.bfloat16,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Online FP8 step: per-token E4M3 quantization of X, then fp8_gemm."""
    _req(X, "X", _FLOATS, ndim=2)
    M, K = X.shape
    _req(qW, "qW", (torch.uint8,), shape=(None, K))
    N = qW.shape[0]
    _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    odt = out.dtype if out is not None else out_dtype
    _out(out, (M, N), odt)
    if workspace is not None:
        _req(workspace, "workspace", (torch.uint8,), ndim=1)
        if workspace.numel() < sq_workspace_bytes(M, K):
            raise ValueError(f"workspace holds {workspace.numel()} bytes; {sq_workspace_bytes(M, K)} needed")
    dev = _place(X=X, qW=qW, w_scale=w_scale, out=out, workspace=workspace)
    out = _alloc(out, (M, N), odt, dev)
    if workspace is None:
        workspace = torch.empty(sq_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    _call("fp8_w8a8_gemm", _ptr(X), _dt(X.dtype), _ptr(qW), _ptr(w_scale), M, N, K, _ptr(out), _dt(out.dtype),
          _ptr(workspace), workspace.numel(), _stream(X))
    return out


# ---------------------------------------------------------------------------
# LLM.int8(): vector-wise INT8 with the outlier feature dimensions multiplied
# in 16-bit.  qW / w_scale are the per-output-channel INT8 weights
# (sq_quantize_weight(W) with no smoothing).
# ---------------------------------------------------------------------------
def _llm_args(X, threshold, max_outliers):
    _req(X, "X", _HALVES, ndim=2)
    M, K = X.shape
    if not threshold >= 0.0:
        raise ValueError(f"threshold must be >= 0, not {threshold}")
    cap = K if max_outliers is None else int(max_outliers)
    if cap < 0:
        raise ValueError(f"max_outliers must be >= 0, not {max_outliers}")
    return M, K, min(cap, K)


def llm_int8_outliers(X: torch.Tensor, threshold: float = 6.0, max_outliers: Optional[int] = None):
    """Outlier detection: -> (factor f32 [K]: +inf for each carved-out column, 1
    otherwise; index int32 [kept] in increasing column order; found).  The
    first `max_outliers` (default K) outlier columns are carved out.
    Synchronizes with the device to read the counts."""
    M, K, cap = _llm_args(X, threshold, max_outliers)
    dev = _place(X=X)
    factor = torch.empty(K, dtype=torch.float32, device=dev)
    index = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    counts = torch.empty(2, dtype=torch.int32, device=dev)
    _call("llm_int8_outliers", _ptr(X), _dt(X.dtype), M, K, float(threshold), cap, _ptr(factor), _ptr(index),
          _ptr(counts), _stream(X))
    kept, found = (int(v) for v in counts.cpu())
    return factor, index[:kept], found


def llm_int8_workspace_bytes(M: int, N: int, K: int, max_outliers: Optional[int] = None) -> int:
    return int(lib().llm_int8_workspace_bytes(M, N, K, K if max_outliers is None else max_outliers))


def llm_int8_gemm(X: torch.Tensor, qW, w_scale, threshold: float = 6.0, max_outliers: Optional[int] = None,
                  out_dtype: torch.dtype = torch.bfloat16, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, n_outliers: Optional[torch.Tensor] = None):
    """Y [M, N] = S_out (X_q qW^T) + X_16 W_16^T: per-token INT8 of the columns of X
    whose largest |x| stays below `threshold`, the others (at most `max_outliers`,
    default K) multiplied in 16-bit.  `n_outliers` (int32 [1], device, optional)
    receives the number of outlier columns found."""
    M, K, cap = _llm_args(X, threshold, max_outliers)
    _req(qW, "qW", (torch.int8,), shape=(None, K))
    N = qW.shape[0]
    _req(w_scale, "w_scale", (torch.float32,), shape=(N,))
    odt = out.dtype if out is not None else out_dtype
    if odt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"out_dtype must be torch.bfloat16 or torch.float32, not {odt}")
    _out(out, (M, N), odt)
    if n_outliers is not None:
        _req(n_outliers, "n_outliers", (torch.int32,), shape=(1,))
    need = llm_int8_workspace_bytes(M, N, K, cap)
    if workspace is not None:
        _req(workspace, "workspace", (torch.uint8,), ndim=1)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes; {need} needed")
    dev = _place(X=X, qW=qW, w_scale=w_scale, out=out, workspace=workspace, n_outliers=n_outliers)
    out = _alloc(out, (M, N), odt, dev)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _call("llm_int8_gemm", _ptr(X), _dt(X.dtype), _ptr(qW), _ptr(w_scale), M, N, K, float(threshold), cap,
          _ptr(out), _dt(out.dtype), _ptr(n_outliers), _ptr(workspace), workspace.numel(), _stream(X))
    return out


# ---------------------------------------------------------------------------
# AWQ scaling search.
# ---------------------------------------------------------------------------
# 0, 0.1, .., 1 as numpy's linspace(0, 1, 11) has them (i * 0.1, the last one
# exactly 1): the grid of the awq listing in "Quantization from Scratch"
AWQ_ALPHAS = tuple(i * 0.1 for i in range(10)) + (1.0,)


def awq_workspace_bytes(N: int, K: int, T: int, n_alpha: int) -> int:
    return int(lib().awq_workspace_bytes(N, K, T, n_alpha))


def awq_search(W: torch.Tensor, X: torch.Tensor, alphas: Sequence[float] = AWQ_ALPHAS,
               workspace: Optional[torch.Tensor] = None):
    """AWQ on 16-bit weights W [N, K] with calibration activations X [T, K] of
    the same type (bf16 or fp16): returns (codes, scales, zeros) of
    W diag(s_best) in the INT4 group-128 format, smooth [K] (= s_best), err
    fp64 [len(alphas)] and best (int64 [1]), all on the device."""
    _req(W, "W", _HALVES, ndim=2)
    N, K = W.shape
    _req(X, "X", (W.dtype,), shape=(None, K))
    T = X.shape[0]
    a = [float(v) for v in alphas]
    if not 1 <= len(a) <= 64:
        raise ValueError(f"takes 1 to 64 alphas, not {len(a)}")
    if not all(0.0 <= v <= 1.0 for v in a):
        raise ValueError(f"alphas must lie in [0, 1]: {a}")
    if K % GROUP != 0:
        raise ValueError(f"K={K} is not a multiple of {GROUP}")
    need = awq_workspace_bytes(N, K, T, len(a))
    if workspace is not None:
        _req(workspace, "workspace", (torch.uint8,), ndim=1)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes; {need} needed")
    dev = _place(W=W, X=X, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // GROUP), dtype=torch.float32, device=dev)
    zeros = torch.empty((N, (K // GROUP + 1) // 2), dtype=torch.uint8, device=dev)
    smooth = torch.empty(K, dtype=torch.float32, device=dev)
    err = torch.empty(len(a), dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int64, device=dev)
    host_alphas = (ctypes.c_double * len(a))(*a)
    _call("awq_search", _ptr(W), _dt(W.dtype), _ptr(X), _dt(X.dtype), N, K, T, ctypes.cast(host_alphas, ctypes.c_void_p),
          len(a), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(smooth), _ptr(err), _ptr(best), _ptr(workspace),
          workspace.numel(), _stream(X))
    return codes, scales, zeros, smooth, err, best


def stream_read(data: torch.Tensor) -> torch.Tensor:
    """Read every byte of a contiguous device tensor once (a plain streaming
    read, for measuring bandwidth); returns the XOR of its 32-bit words as a
    uint32-valued int32 tensor [1] on the device."""
    if not isinstance(data, torch.Tensor):
        raise ValueError("data must be a torch.Tensor")
    nbytes = data.numel() * data.element_size()
    if nbytes == 0 or nbytes % 16 != 0:
        raise ValueError(f"data must hold a positive multiple of 16 bytes, not {nbytes}")
    dev = _place(data=data)
    out = torch.empty(1, dtype=torch.int32, device=dev)
    _call("qmm_stream_read", _ptr(data), nbytes, _ptr(out), _stream(data))
    return out
