"""Helpers for the GPU parity tests (comparison rules and seeded operands)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Floating-point outputs of the matmuls are compared with the oracle's fp64
# value elementwise:
#   |y - y_ref| <= RTOL * |y_ref| + RTOL * rms(y_ref) + half an ulp of the output dtype,
# RTOL = 1e-3 (fp32 accumulation).  The rms term keeps outputs that cancel to
# nearly zero from failing on absolute noise; the ulp term is the rounding of
# the result to a 16-bit output type (2^-9 relative for bf16, 2^-12 for fp16).
RTOL = 1e-3
OUT_HALF_ULP = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, file=sys.stderr, flush=True)


def assert_close(y: torch.Tensor, y_ref: np.ndarray, what: str, normwise: float = 1e-5) -> float:
    """Check the elementwise rule above; also the norm-wise relative error of
    fp32 outputs (expected ~1e-7) against `normwise`.  Returns the latter."""
    out_dt = y.dtype
    yv = y.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(y_ref, np.float64).reshape(yv.shape)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = RTOL * np.abs(ref) + RTOL * rms + OUT_HALF_ULP[out_dt] * np.abs(ref)
    err = np.abs(yv - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at {i}: "
                             f"got {yv[i]!r} want {ref[i]!r} bound {bound[i]!r}")
    rel = float(np.linalg.norm(yv - ref) / max(np.linalg.norm(ref), 1e-300))
    if out_dt == torch.float32:
        assert rel < normwise, f"{what}: norm-wise relative error {rel:.3e}"
    return rel


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype.itemsize == b.dtype.itemsize and \
        np.array_equal(a.view(np.uint8), b.view(np.uint8))


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    d = np.nonzero(a.reshape(-1).view(np.uint8) != b.reshape(-1).view(np.uint8))[0]
    if d.size == 0:
        return "none"
    i = d[0] // a.dtype.itemsize
    return f"{d.size} bytes differ; first element {np.unravel_index(i, a.shape)}: {a.reshape(-1)[i]!r} vs {b.reshape(-1)[i]!r}"


def random_w4(n: int, k: int, seed: int):
    """Arbitrary INT4 operands (codes, scales, zero-points), not produced by a quantizer."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    z = g.integers(0, 16, size=(n, k // 128)).astype(np.uint8)
    s = (g.random((n, k // 128), dtype=np.float32) * np.float32(0.01) + np.float32(1e-4)).astype(np.float32)
    return q, s, z


def stratified_rows(n: int, block: int) -> np.ndarray:
    """One row in every block of `block` consecutive rows, its position in the
    block cycling through 0..block-1, so a sample meets every output tile of
    that height (and, across tiles, every position within one)."""
    starts = np.arange(0, n, block)
    return np.minimum(starts + (np.arange(len(starts)) % block), n - 1)
