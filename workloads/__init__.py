"""Seeded synthetic inputs for the quantizer and the quantized matmuls.

This module only draws random numbers and rounds them once to the storage
dtype. It holds none of the quantization arithmetic, so both the CPU oracle
(test infrastructure under ``oracle/``) and the HIP path can be fed from it
without sharing any of the method's code.

Recipe (one ``numpy.random.Generator(PCG64(1000 * workload_id + stream))``
per stream; stream 0 = weights, 1 = activations, 2 = outlier positions):

* weights are ``float32 standard_normal * sigma``;
* planted outliers are applied in float32;
* the tensor is then rounded ONCE to its storage dtype (bf16 / fp16 by
  round-to-nearest-even through torch's CPU cast); that rounded tensor is the
  input of record for both sides.

The shapes and distributions follow the workloads the pages reason about:
LLM linear layers (Llama-7B-like 4096x4096 / 11008x4096, a 14336x4096 MLP
projection, 70B-class 28672x8192 / 8192x28672 MLP slices), Gaussian weights
with a few large entries, and activations with a handful of outlier channels
(the activation-outlier sections of "How quantization works" and of
"Quantization" (Engine Room ch. 15)).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

__all__ = [
    "rng", "gaussian", "plant_replace", "plant_scale_entries", "plant_scale_columns",
    "to_dtype", "WORKLOADS", "Workload", "weight", "activations", "sq_activations",
]


def rng(workload_id: int, stream: int) -> np.random.Generator:
    """The generator for (workload, stream)."""
    return np.random.Generator(np.random.PCG64(1000 * int(workload_id) + int(stream)))


def gaussian(g: np.random.Generator, shape: Tuple[int, ...], sigma: float) -> np.ndarray:
    """float32 N(0, sigma^2) samples."""
    a = g.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def plant_replace(a: np.ndarray, g: np.random.Generator, count: int, magnitude: float) -> np.ndarray:
    """Replace `count` seeded distinct entries by +-magnitude (seeded signs)."""
    flat = a.reshape(-1)
    pos = g.choice(flat.size, size=count, replace=False)
    sign = np.where(g.integers(0, 2, size=count) == 0, -1.0, 1.0).astype(np.float32)
    flat[pos] = sign * np.float32(magnitude)
    return pos


def plant_scale_entries(a: np.ndarray, g: np.random.Generator, fraction: float, factor: float) -> np.ndarray:
    """Multiply round(fraction * size) seeded distinct entries by `factor` (float32)."""
    flat = a.reshape(-1)
    count = int(round(fraction * flat.size))
    pos = g.choice(flat.size, size=count, replace=False)
    flat[pos] *= np.float32(factor)
    return pos


def plant_scale_columns(a: np.ndarray, g: np.random.Generator, count: int, lo: float, hi: float) -> np.ndarray:
    """Multiply `count` seeded distinct columns by linspace(lo, hi, count)."""
    cols = g.choice(a.shape[1], size=count, replace=False)
    factors = np.linspace(lo, hi, count).astype(np.float32)
    a[:, cols] *= factors[None, :]
    return cols


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    """One round-to-nearest-even cast of a float32 array to the storage dtype (CPU tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == "f32" else t.to(_TORCH_DT[dtype])


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                       # seed base
    name: str
    weights: Tuple[Tuple[int, int], ...]   # (N, K) of each weight matrix
    w_dtype: str
    w_sigma: float
    x_dtype: str
    batches: Tuple[int, ...]       # activation rows per matmul
    outliers: str                  # "replace4" | "scale0.1%" | "none"
    note: str


# The six workloads (sizes, dtypes and distributions as stated for each).
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(1, "single 512x512 fp32 weight with 4 planted +-0.5 outliers; fp16 GEMV x[1,512]",
                     ((512, 512),), "f32", 0.02, "f16", (1,), "replace4", ""),
    "llama7b": Workload(2, "Llama-7B-like decode layer: bf16 4096x4096 and 11008x4096, 0.1% entries x10; GEMV B=1",
                        ((4096, 4096), (11008, 4096)), "bf16", 0.02, "bf16", (1,), "scale0.1%", ""),
    "gemm": Workload(3, "batched W4A16 GEMM: 14336x4096 INT4 G128, bf16 X of M in {16,64,256} tokens",
                     ((14336, 4096),), "bf16", 0.02, "bf16", (16, 64, 256), "none", ""),
    "smoothquant": Workload(4, "SmoothQuant W8A8: X 2048x4096 bf16 with 6 outlier channels x50..100, W 4096x4096",
                            ((4096, 4096),), "bf16", 0.02, "bf16", (2048,), "none", ""),
    "awq": Workload(6, "AWQ scaling search: bf16 W 4096x4096; calibration X 2048x4096 bf16, 1% of the channels x4..x58",
                    ((4096, 4096),), "bf16", 0.02, "bf16", (2048,), "none", ""),
    "mlp70b": Workload(5, "70B-class MLP decode: bf16 28672x8192 and 8192x28672, 0.1% entries x10; GEMV B=1 and B=8",
                       ((28672, 8192), (8192, 28672)), "bf16", 0.015, "bf16", (1, 8), "scale0.1%", ""),
}


def weight(wl: Workload, index: int = 0, shape: Optional[Tuple[int, int]] = None) -> Tuple[torch.Tensor, np.ndarray]:
    """Weight matrix `index` of a workload, rounded to its storage dtype.

    `shape` overrides the size (same recipe, used for small parity cases).
    Returns (CPU tensor in storage dtype, outlier positions)."""
    n, k = shape if shape is not None else wl.weights[index]
    g = rng(wl.wid, 0 + 10 * index)
    w = gaussian(g, (n, k), wl.w_sigma)
    go = rng(wl.wid, 2 + 10 * index)
    if wl.outliers == "replace4":
        pos = plant_replace(w, go, 4, 0.5)
    elif wl.outliers == "scale0.1%":
        pos = plant_scale_entries(w, go, 0.001, 10.0)
    else:
        pos = np.zeros(0, dtype=np.int64)
    return to_dtype(w, wl.w_dtype), pos


def activations(wl: Workload, m: int, k: int, salt: int = 0) -> torch.Tensor:
    """Activation matrix [m, k] ~ N(0, 1) in the workload's activation dtype."""
    g = rng(wl.wid, 1 + 10 * salt)
    return to_dtype(gaussian(g, (m, k), 1.0), wl.x_dtype)


def sq_activations(wl: Workload, m: int, k: int, n_channels: int = 6,
                   lo: float = 50.0, hi: float = 100.0) -> Tuple[torch.Tensor, np.ndarray]:
    """Activations N(0,1) with `n_channels` seeded outlier channels scaled linspace(lo, hi)."""
    g = rng(wl.wid, 1)
    x = gaussian(g, (m, k), 1.0)
    cols = plant_scale_columns(x, rng(wl.wid, 2), min(n_channels, k), lo, hi)
    return to_dtype(x, wl.x_dtype), cols


def uniform_ints(seed: int, shape: Tuple[int, ...], lo: int, hi: int) -> np.ndarray:
    """Seeded integers in [lo, hi] (inclusive), for raw code / int8 test operands."""
    return np.random.Generator(np.random.PCG64(seed)).integers(lo, hi + 1, size=shape)


def shapes_for_parity() -> List[Tuple[int, int]]:
    """Small (N, K) cases spanning several tiles plus ragged tails in N and K."""
    return [(1, 128), (3, 384), (17, 640), (64, 1152), (129, 2176), (257, 4224)]
