#!/usr/bin/env python3
"""Benchmark of the INT4 / INT8 quantized-matmul hot path on one MI355X.

One step runs every stage of the path once, on synthetic seeded inputs that
are resident in HBM before timing starts, for all six workloads:

  70B-class MLP, bf16 weights 28672x8192 and 8192x28672 (N(0, 0.015), 0.1% of
  entries x10): quantize_groupwise on both, quantize_groupwise_symmetric on
  the first, dequantize to bf16 on both;
  single 512x512 fp32 weight (4 planted +-0.5 outliers): quantize, then the
  fp16 B=1 GEMV;
  Llama-7B-like decode layer, bf16 4096x4096 and 11008x4096: quantize both,
  then the B=1 GEMV on both;
  batched W4A16 GEMM, bf16 14336x4096: quantize, then X bf16 [M, 4096] for
  M = 16, 64, 256;
  SmoothQuant W8A8, X 2048x4096 (6 outlier channels x50..100), W 4096x4096:
  sq_smooth_factors, sq_quantize_weight, per-tensor activation quantization
  (the W8A8 baseline: X read twice), sq_int8_gemm alone (i8-MFMA GEMM and
  rescale to bf16, on activations quantized before timing) and
  smooth_quant_w8a8_gemm (per-token smoothing + INT8 quantization, then the
  same GEMM); FP8 E4M3 W8A8 on the same shapes: fp8_quantize of the weights,
  fp8_gemm alone and the online fp8_w8a8_gemm; LLM.int8() (llm_int8_gemm,
  outlier threshold 6) on the same shapes;
  AWQ's scaling search (awq_search) on a bf16 4096x4096 layer with 2048
  calibration tokens (1% of the channels x4..x58) over the 11-point alpha grid;
  70B-class MLP decode: w4a16_gemv B=8 then B=1 on both matrices (B=1 is the
  headline), then weight-only INT8 (w8a16_gemv) at B=1 and B=8;
  stored-format variants on the 28672x8192 matrix (binary16 scales, groups of
  32 and 1024, 3- and 8-bit codes): quantize_groupwise_ex and the B=1
  wxa16_gemv.

Cache: the last-level cache is 256 MB.  No op reads an operand that anything
touched within the last 512 MB of traffic: every op reads buffers of its own
(the packed 70B weights exist in 4 copies per matrix, the 14336x4096 weight in
3, the Llama-7B-like and 512x512 ones in 2, the SmoothQuant operands in one
copy per reading op) and the copies rotate between steps.  The bench computes
each op's reuse distance from this bookkeeping (bytes of algorithmic traffic
since any of its inputs was last touched, over a steady-state run of steps),
reports it per op (`reuse_MB`) and fails if an HBM-bound op falls under
512 MB.

Timing: every op is bracketed by events on the stream it runs on (the
library launches on torch's current stream), created without the system
fence so that recording them leaves the caches alone; the two B=1 GEMVs of
the 70B matrices run back to back inside one event pair and share its time.
`value` is their effective bandwidth: algorithmic bytes (packed codes,
scales, zero-points, activations in, outputs out) over kernel time.  Each
op's breakdown entry gives the mean, median, p10 and p90 over the timed
steps; `config.plain_read_GBps` is a plain 1 GiB streaming read (the
library's `qmm_stream_read`, after the timed steps), as context for the HBM
fractions, and `config.vendor_library_gemms` the ROCm BLAS libraries' INT8
and bf16 GEMM rates at 2048x4096x4096 (through torch), as context for the
MFMA fractions.  `config.headline_after_flush` times the two B=1 GEMVs
again after the timed steps, each pair right after a 1 GiB read with
ordinary (cache-allocating) loads, as a check that the headline is not
served from the last-level cache.

CPU baseline: the plain C oracle's reference for the same B=1 GEMVs
(dequantize + fp64 product), single-threaded, and its OpenMP build over all
the threads the host grants (OMP_NUM_THREADS); both on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_matmul_quantize_amd as qmm  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # dense bf16 MFMA, published
I8_PEAK_TOPS = 5000.0           # dense int8 MFMA, published
FP8_PEAK_TFLOPS = 5000.0        # dense fp8 MFMA, published
COLD_BYTES = 512e6              # twice the 256 MB last-level cache
COPIES_70B = 4


class HipEvent:
    """A HIP timing event on torch's current stream, created with
    hipEventDisableSystemFence: recording it does not write back and
    invalidate the caches (which a default event does, adding microseconds to
    the next kernel).  Read only after a device synchronize."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        if HipEvent._hip is None:
            import ctypes
            HipEvent._ct = ctypes
            # the runtime torch already loaded (same SONAME), so streams match
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        ct = HipEvent._ct
        self.h = ct.c_void_p()
        st = HipEvent._hip.hipEventCreateWithFlags(ct.byref(self.h), ct.c_uint(self.DISABLE_SYSTEM_FENCE))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")

    def record(self):
        ct = HipEvent._ct
        st = HipEvent._hip.hipEventRecord(self.h, ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_time(self, end):
        ct = HipEvent._ct
        ms = ct.c_float()
        st = HipEvent._hip.hipEventElapsedTime(ct.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value


def decode_step_ms(params, batch, bytes_per_weight, bandwidth, flops):
    """Roofline time of one decode step ("Quantization from Scratch", "What it
    buys at decode"): every weight is read once from memory and each does 2
    flops per sequence in the batch; the step takes the longer of the two."""
    return max(params * bytes_per_weight / bandwidth, 2.0 * params * batch / flops) * 1e3


def matmul_bound(tokens, bytes_per_weight, bandwidth=HBM_PEAK_GBPS * 1e9, flops=BF16_PEAK_TFLOPS * 1e12):
    """'hbm' while reading the weights takes longer than the matrix work on
    `tokens` tokens (below the ridge of the roofline), else 'mfma'."""
    return "hbm" if 2.0 * tokens / bytes_per_weight < flops / bandwidth else "mfma"


def w4_kernel_name(M, N, dev):
    """Which W4A16 kernel the library picks for M tokens and N weight rows
    (the rule in w4a16.hip's launchers), for labelling only."""
    if M <= 2:
        return "gemv_valu_kernel"
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    cdiv = lambda a, b: -(-a // b)
    mt = cdiv(M, 16)
    if M <= 64 and (mt * cdiv(N, 64) >= cus or 2 * mt * cdiv(N, 32) >= 3 * cus):
        return "w4_rows_kernel"
    if M <= 16:
        return "w4_lds_kernel"
    if M > 32 and cdiv(M, 64) * cdiv(N, 128) >= cus:
        return "w4_tile_kernel"
    return "w4_lds_kernel"


def w8_kernel_name(B, K):
    """w8a16_gemv's dispatch: vector ALUs for one or two tokens, matrix cores
    from three (LDS-staged weights when K is a multiple of 256)."""
    if B <= 2:
        return "w8_gemv_kernel"
    return "w8_lds_kernel" if K % 256 == 0 else "w8_mfma_kernel"


def w4_bytes(n, k):
    c, s, z = qmm.w4_sizes(n, k)
    return c + s + z


# Stored-format variants timed on the 28672x8192 matrix: (tag, group, bits, scale dtype).
VARIANTS = [("g128-4bit-f16scale", 128, 4, torch.float16), ("g32-4bit", 32, 4, torch.float32),
            ("g1024-4bit", 1024, 4, torch.float32), ("g128-3bit-f16scale", 128, 3, torch.float16),
            ("g128-8bit-f16scale", 128, 8, torch.float16)]


def fmt_bytes(n, k, f):
    c, s, z = qmm.wq_sizes(n, k, f["group"], f["bits"], f["sdt"])
    return c + s + z


def P(t):
    return qmm._ptr(t)


def S(t):
    return qmm._stream(t)


def ok(st):
    assert st == 0, qmm.lib().qmm_status_string(st).decode()


class Ops:
    """The ordered ops of one step plus the buffers each reads and writes."""

    def __init__(self):
        self.ops = []

    def add(self, name, fn, nbytes, bound, kernel, config, reads, writes=lambda i: [], flops=0, peak=None,
            group=None):
        self.ops.append(dict(name=name, fn=fn, bytes=nbytes, bound=bound, kernel=kernel, config=config,
                             reads=reads, writes=writes, flops=flops, peak=peak, group=group))

    def reuse_distances(self, steps=12, settle=4):
        """Minimum over steady-state steps of the algorithmic traffic between
        the last touch of any input of an op and the op itself."""
        pos, last = 0, {}
        dmin = {op["name"]: float("inf") for op in self.ops}
        for i in range(steps):
            for op in self.ops:
                for b in op["reads"](i):
                    if i >= settle and b in last:
                        dmin[op["name"]] = min(dmin[op["name"]], pos - last[b])
                pos += op["bytes"]
                for b in list(op["reads"](i)) + list(op["writes"](i)):
                    last[b] = pos
        return dmin


def quant_op(ops, lib, name, w, dt, n, k, outs, cfg, wkey, okey, kernel, sym=False):
    """quantize_groupwise(_symmetric) of w into outs[i % len(outs)]."""
    fn_c = lib.quantize_groupwise_symmetric if sym else lib.quantize_groupwise
    elem = 4 if dt == qmm.F32 else 2

    def run(i):
        c, s, z = outs[i % len(outs)]
        ok(fn_c(P(w), dt, n, k, 128, 4, P(c), P(s), P(z), S(w)))
    ops.add(name, run, n * k * elem + w4_bytes(n, k), "hbm", kernel, cfg, reads=lambda i: [wkey],
            writes=lambda i: [f"{okey}[{i % len(outs)}]"])


def gemv_op(ops, lib, name, copies, sel, okey, n, k, x, y, B, xdt, cfg, xkey, group=None):
    """w4a16_gemv on copy sel(i) of the packed weight."""
    def run(i):
        c, s, z = copies[sel(i)]
        ok(lib.w4a16_gemv(P(c), P(s), P(z), n, k, 128, P(x), xdt, B, P(y), xdt, S(x)))
    ops.add(name, run, w4_bytes(n, k) + B * k * 2 + B * n * 2, "hbm", w4_kernel_name(B, n, x.device), cfg,
            reads=lambda i: [f"{okey}[{sel(i)}]", xkey], flops=2 * B * n * k, group=group)


def build_ops(dev):
    """Allocate every input/output and return the ordered list of timed ops."""
    lib = qmm.lib()
    ops = Ops()

    # ---- 70B-class MLP matrices: quantizers and dequantizer ----------------
    wl5 = workloads.WORKLOADS["mlp70b"]
    mats = []
    for idx, (n, k) in enumerate(wl5.weights):
        w_cpu, _ = workloads.weight(wl5, idx)
        w = w_cpu.to(dev)
        del w_cpu
        copies = [qmm.quantize_groupwise(w) for _ in range(COPIES_70B)]
        mats.append(dict(idx=idx, n=n, k=k, w=w, copies=copies, key=f"w4_70b{idx}"))
    cfg5 = "70B-class MLP decode"
    C = COPIES_70B
    # copy use per step i: the quantizer writes i%4, the dequantizer reads
    # (i+3)%4, the B=8 GEMV (i+1)%4 and the B=1 GEMV (i+2)%4, so between two
    # uses of a copy there is at least a whole step of other traffic
    for m in mats:
        quant_op(ops, lib, f"quantize {m['n']}x{m['k']}", m["w"], qmm.BF16, m["n"], m["k"], m["copies"], cfg5,
                 f"bf16_70b{m['idx']}", m["key"], "quantize_g128_lds_kernel")
    m0 = mats[0]
    sym_out = [qmm.quantize_groupwise(m0["w"], symmetric=True)]
    quant_op(ops, lib, f"quantize_symmetric {m0['n']}x{m0['k']}", m0["w"], qmm.BF16, m0["n"], m0["k"], sym_out, cfg5,
             "bf16_70b0", "sym_70b0", "quantize_g128_lds_kernel (symmetric)", sym=True)
    for m in mats:
        m["what"] = torch.empty((m["n"], m["k"]), dtype=torch.bfloat16, device=dev)

        def deq(i, m=m):
            c, s, z = m["copies"][(i + 3) % C]
            ok(lib.dequantize(P(c), P(s), P(z), m["n"], m["k"], 128, 4, P(m["what"]), qmm.BF16, S(c)))
        ops.add(f"dequantize {m['n']}x{m['k']}", deq, w4_bytes(m["n"], m["k"]) + m["n"] * m["k"] * 2, "hbm",
                "dequantize_g128_kernel", cfg5, reads=lambda i, m=m: [f"{m['key']}[{(i + 3) % C}]"],
                writes=lambda i, m=m: [f"what_70b{m['idx']}"])

    # ---- stored-format variants on the 28672x8192 matrix ---------------------
    # quantizer writes copy i%2, the B=1 GEMV (at the end of the step) reads (i+1)%2
    # the variant quantizers read two further copies of the bf16 weights in turn
    w0c = [m0["w"].clone() for _ in range(2)]
    fmts = []
    for tag, group, bits, sdt in VARIANTS:
        cps = [qmm.quantize_groupwise_ex(m0["w"], group, bits, sdt) for _ in range(2)]
        fmts.append(dict(tag=tag, group=group, bits=bits, sdt=sdt, copies=cps, key=f"fmt_{tag}",
                         x=workloads.activations(wl5, 1, m0["k"], salt=0).to(dev),
                         y=torch.empty((1, m0["n"]), dtype=torch.bfloat16, device=dev)))
    for j, f in enumerate(fmts):
        def quant_fmt(i, f=f, m=m0, w=w0c[j % 2]):
            c, sc, z = f["copies"][i % 2]
            ok(lib.quantize_groupwise_ex(P(w), qmm.BF16, m["n"], m["k"], f["group"], f["bits"], qmm._sdt(f["sdt"]),
                                         0, P(c), P(sc), P(z), S(w)))
        ops.add(f"quantize_ex {f['tag']} {m0['n']}x{m0['k']}", quant_fmt,
                m0["n"] * m0["k"] * 2 + fmt_bytes(m0["n"], m0["k"], f), "hbm", "quantize_fmt_kernel", cfg5,
                reads=lambda i, j=j: [f"bf16_70b0_copy{j % 2}"], writes=lambda i, f=f: [f"{f['key']}[{i % 2}]"])

    # ---- single 512x512 fp32 weight: quantize, fp16 GEMV --------------------
    wl1 = workloads.WORKLOADS["tiny"]
    n1, k1 = wl1.weights[0]
    w1 = workloads.weight(wl1, 0)[0].to(dev)
    c1 = [qmm.quantize_groupwise(w1) for _ in range(2)]
    x1 = workloads.activations(wl1, 1, k1).to(dev)
    y1 = torch.empty((1, n1), dtype=torch.float16, device=dev)
    cfg1 = "single 512x512 fp32 weight"
    quant_op(ops, lib, f"quantize {n1}x{k1} fp32", w1, qmm.F32, n1, k1, c1, cfg1, "f32_tiny", "w4_tiny",
             "quantize_g128_flat_kernel")
    gemv_op(ops, lib, f"w4a16_gemv B=1 {n1}x{k1} fp16", c1, lambda i: (i + 1) % 2, "w4_tiny", n1, k1, x1, y1, 1,
            qmm.F16, cfg1, "x_tiny")

    # ---- Llama-7B-like decode layer: quantize, B=1 GEMV ----------------------
    wl2 = workloads.WORKLOADS["llama7b"]
    l7 = []
    for idx, (n, k) in enumerate(wl2.weights):
        w = workloads.weight(wl2, idx)[0].to(dev)
        l7.append(dict(idx=idx, n=n, k=k, w=w, copies=[qmm.quantize_groupwise(w) for _ in range(2)],
                       x=workloads.activations(wl2, 1, k, salt=idx).to(dev),
                       y=torch.empty((1, n), dtype=torch.bfloat16, device=dev)))
    cfg2 = "Llama-7B-like decode layer"
    for m in l7:
        quant_op(ops, lib, f"quantize {m['n']}x{m['k']}", m["w"], qmm.BF16, m["n"], m["k"], m["copies"], cfg2,
                 f"bf16_l7{m['idx']}", f"w4_l7{m['idx']}", "quantize_g128_lds_kernel")
    for m in l7:
        gemv_op(ops, lib, f"w4a16_gemv B=1 {m['n']}x{m['k']}", m["copies"], lambda i: (i + 1) % 2,
                f"w4_l7{m['idx']}", m["n"], m["k"], m["x"], m["y"], 1, qmm.BF16, cfg2, f"x_l7{m['idx']}")

    # ---- batched W4A16 GEMM: quantize, M = 16 / 64 / 256 ---------------------
    wl3 = workloads.WORKLOADS["gemm"]
    n3, k3 = wl3.weights[0]
    w3 = workloads.weight(wl3, 0)[0].to(dev)
    g3 = [qmm.quantize_groupwise(w3) for _ in range(3)]
    q3 = [qmm.quantize_groupwise(w3)]
    cfg3 = "batched W4A16 GEMM 14336x4096"
    quant_op(ops, lib, f"quantize {n3}x{k3}", w3, qmm.BF16, n3, k3, q3, cfg3, "bf16_gemm", "w4_gemm_q",
             "quantize_g128_lds_kernel")
    for j, M in enumerate(wl3.batches):
        X = workloads.activations(wl3, M, k3).to(dev)
        Y = torch.empty((M, n3), dtype=torch.bfloat16, device=dev)

        def gemm(i, X=X, Y=Y, M=M, j=j):
            c, s, z = g3[(i + j) % 3]
            ok(lib.w4a16_gemm(P(c), P(s), P(z), n3, k3, 128, P(X), qmm.BF16, M, P(Y), qmm.BF16, S(X)))
        ops.add(f"w4a16_gemm M={M} {n3}x{k3}", gemm, w4_bytes(n3, k3) + M * k3 * 2 + M * n3 * 2,
                matmul_bound(M, w4_bytes(n3, k3) / (n3 * k3)), w4_kernel_name(M, n3, dev), cfg3,
                reads=lambda i, j=j, M=M: [f"w4_gemm[{(i + j) % 3}]", f"x_gemm{M}"], flops=2 * M * n3 * k3)

    # ---- SmoothQuant W8A8 ---------------------------------------------------
    wl4 = workloads.WORKLOADS["smoothquant"]
    n4, k4 = wl4.weights[0]
    m4 = wl4.batches[0]
    x4c, _ = workloads.sq_activations(wl4, m4, k4)
    w4c, _ = workloads.weight(wl4, 0)
    x4 = [x4c.to(dev) for _ in range(3)]        # factors, per-tensor quantizer, online call
    w4 = [w4c.to(dev) for _ in range(2)]        # factors, weight quantizer
    cfg4 = "SmoothQuant W8A8 2048x4096x4096"
    smooth = torch.empty(k4, dtype=torch.float32, device=dev)
    cx, cw = torch.empty_like(smooth), torch.empty_like(smooth)
    ok(lib.sq_smooth_factors(P(x4[0]), qmm.BF16, m4, P(w4[0]), qmm.BF16, n4, k4, 0.5, P(cx), P(cw), P(smooth),
                             S(x4[0])))
    # each reader of the smoothing factors has its own copy of them
    sm_w, sm_a, sm_o = smooth.clone(), smooth.clone(), smooth.clone()
    qw_out = torch.empty((n4, k4), dtype=torch.int8, device=dev)
    wsc_out = torch.empty(n4, dtype=torch.float32, device=dev)
    qw_a, wsc_a = qmm.sq_quantize_weight(w4[1], smooth)        # read by the INT8 GEMM alone
    qw_b, wsc_b = qmm.sq_quantize_weight(w4[1], smooth)        # read by the online call
    qx_pre, xsc_pre = qmm.sq_quantize_activation(x4[0], smooth)
    qx_t = torch.empty((m4, k4), dtype=torch.int8, device=dev)
    xsc_t = torch.empty(m4, dtype=torch.float32, device=dev)
    y4a = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    y4b = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qmm.sq_workspace_bytes(m4, k4), dtype=torch.uint8, device=dev)

    def sq_factors(i):
        ok(lib.sq_smooth_factors(P(x4[0]), qmm.BF16, m4, P(w4[0]), qmm.BF16, n4, k4, 0.5, P(cx), P(cw), P(smooth),
                                 S(x4[0])))

    def sq_weight(i):
        ok(lib.sq_quantize_weight(P(w4[1]), qmm.BF16, P(sm_w), n4, k4, P(qw_out), P(wsc_out), S(w4[1])))

    def sq_act_tensor(i):
        ok(lib.sq_quantize_activation_per_tensor(P(x4[1]), qmm.BF16, P(sm_a), m4, k4, P(qx_t), P(xsc_t),
                                                 S(x4[1])))

    def sq_gemm(i):
        ok(lib.sq_int8_gemm(P(qx_pre), P(xsc_pre), P(qw_a), P(wsc_a), m4, n4, k4, P(y4a), qmm.BF16, S(qx_pre)))

    def sq_online(i):
        ok(lib.smooth_quant_w8a8_gemm(P(x4[2]), qmm.BF16, P(sm_o), P(qw_b), P(wsc_b), m4, n4, k4, P(y4b), qmm.BF16,
                                      P(ws), ws.numel(), S(x4[2])))

    ops.add(f"sq_smooth_factors {m4}x{k4} / {n4}x{k4}", sq_factors, (m4 + n4) * k4 * 2 + 3 * k4 * 4, "hbm",
            "colmax2_kernel + smooth_finalize_kernel", cfg4, reads=lambda i: ["x4[0]", "w4[0]"],
            writes=lambda i: ["smooth"])
    ops.add(f"sq_quantize_weight {n4}x{k4}", sq_weight, n4 * k4 * 3 + k4 * 4 + n4 * 4, "hbm", "rowquant8_kernel",
            cfg4, reads=lambda i: ["w4[1]", "sm_w"], writes=lambda i: ["qw_out"])
    ops.add(f"sq_quantize_activation_per_tensor {m4}x{k4}", sq_act_tensor,
            2 * m4 * k4 * 2 + k4 * 4 + m4 * k4 + m4 * 4, "hbm", "rowquant8_kernel x2 + tensor_scale_kernel", cfg4,
            reads=lambda i: ["x4[1]", "sm_a"], writes=lambda i: ["qx_t"])
    ops.add(f"sq_int8_gemm {m4}x{n4}x{k4}", sq_gemm, m4 * k4 + m4 * 4 + n4 * k4 + n4 * 4 + m4 * n4 * 2, "mfma",
            "i8_gemm_kernel", cfg4, reads=lambda i: ["qx_pre", "qw_a"], writes=lambda i: ["y4a"],
            flops=2 * m4 * n4 * k4, peak=I8_PEAK_TOPS)
    ops.add(f"smooth_quant_w8a8_gemm {m4}x{n4}x{k4}", sq_online,
            m4 * k4 * 2 + k4 * 4 + (m4 * k4 + m4 * 4) * 2 + n4 * k4 + n4 * 4 + m4 * n4 * 2, "mfma",
            "rowquant8_kernel + i8_gemm_kernel", cfg4, reads=lambda i: ["x4[2]", "qw_b", "sm_o"],
            writes=lambda i: ["y4b"], flops=2 * m4 * n4 * k4, peak=I8_PEAK_TOPS)

    # ---- FP8 E4M3 W8A8 on the same shapes ------------------------------------
    x8in = x4c.to(dev)                           # the online FP8 call's activations
    w8in = w4c.to(dev)                           # the FP8 weight quantizer's input
    q8w, s8w = qmm.fp8_quantize(w4[1])           # read by the FP8 GEMM alone
    q8wb, s8wb = qmm.fp8_quantize(w4[1])         # read by the online FP8 call
    q8x, s8x = qmm.fp8_quantize(x4[0])
    q8w_out = torch.empty((n4, k4), dtype=torch.uint8, device=dev)
    s8w_out = torch.empty(n4, dtype=torch.float32, device=dev)
    y8a = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    y8b = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    ws8 = torch.empty(qmm.sq_workspace_bytes(m4, k4), dtype=torch.uint8, device=dev)
    cfg4f = "FP8 E4M3 W8A8 2048x4096x4096"

    def fp8_wq(i):
        ok(lib.fp8_quantize(P(w8in), qmm.BF16, n4, k4, 0, P(q8w_out), P(s8w_out), S(w8in)))

    def fp8_mm(i):
        ok(lib.fp8_gemm(P(q8x), P(s8x), P(q8w), P(s8w), m4, n4, k4, P(y8a), qmm.BF16, S(q8x)))

    def fp8_online(i):
        ok(lib.fp8_w8a8_gemm(P(x8in), qmm.BF16, P(q8wb), P(s8wb), m4, n4, k4, P(y8b), qmm.BF16, P(ws8), ws8.numel(),
                             S(x8in)))

    ops.add(f"fp8_quantize weights {n4}x{k4}", fp8_wq, n4 * k4 * 3 + n4 * 4, "hbm", "rowquant8_kernel (E4M3)", cfg4f,
            reads=lambda i: ["w8in"], writes=lambda i: ["q8w_out"])
    ops.add(f"fp8_gemm {m4}x{n4}x{k4}", fp8_mm, m4 * k4 + m4 * 4 + n4 * k4 + n4 * 4 + m4 * n4 * 2, "mfma",
            "i8_gemm_kernel (fp8)", cfg4f, reads=lambda i: ["q8x", "q8w"], writes=lambda i: ["y8a"],
            flops=2 * m4 * n4 * k4, peak=FP8_PEAK_TFLOPS)
    ops.add(f"fp8_w8a8_gemm {m4}x{n4}x{k4}", fp8_online,
            m4 * k4 * 2 + (m4 * k4 + m4 * 4) * 2 + n4 * k4 + n4 * 4 + m4 * n4 * 2, "mfma",
            "rowquant8_kernel (E4M3) + i8_gemm_kernel (fp8)", cfg4f, reads=lambda i: ["x8in", "q8wb"],
            writes=lambda i: ["y8b"], flops=2 * m4 * n4 * k4, peak=FP8_PEAK_TFLOPS)

    # ---- LLM.int8() on the same shapes (outlier threshold 6: the six planted
    # channels are carved out) -------------------------------------------------
    xl = x4c.to(dev)                             # the LLM.int8() call's activations
    qw_l, wsc_l = qmm.sq_quantize_weight(w4[1])  # per-output-channel INT8, no smoothing
    yl = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    wsl = torch.empty(qmm.llm_int8_workspace_bytes(m4, n4, k4), dtype=torch.uint8, device=dev)
    nl = torch.zeros(1, dtype=torch.int32, device=dev)
    cfg4l = "LLM.int8() 2048x4096x4096, outlier threshold 6"

    def llm_int8(i):
        ok(lib.llm_int8_gemm(P(xl), qmm.BF16, P(qw_l), P(wsc_l), m4, n4, k4, 6.0, k4, P(yl), qmm.BF16, P(nl),
                             P(wsl), wsl.numel(), S(xl)))

    ops.add(f"llm_int8_gemm {m4}x{n4}x{k4}", llm_int8,
            2 * m4 * k4 * 2 + 3 * k4 * 4 + (m4 * k4 + m4 * 4) * 2 + n4 * k4 + n4 * 4 + m4 * n4 * 2, "mfma",
            "colmax2_kernel + outlier_select_kernel + rowquant8_kernel + outlier_gather_kernel + "
            "i8_gemm_kernel (outlier epilogue)", cfg4l, reads=lambda i: ["xl", "qw_l"], writes=lambda i: ["yl"],
            flops=2 * m4 * n4 * k4, peak=I8_PEAK_TOPS)

    # ---- AWQ's scaling search: one 4096x4096 layer, 2048 calibration tokens
    # with 1% of the channels scaled x4..x58, the 11-point alpha grid --------
    wla = workloads.WORKLOADS["awq"]
    na, ka = wla.weights[0]
    ta = wla.batches[0]
    wa = workloads.weight(wla)[0].to(dev)
    xa = workloads.sq_activations(wla, ta, ka, n_channels=ka // 100, lo=4.0, hi=58.0)[0].to(dev)
    n_al = len(qmm.AWQ_ALPHAS)
    alphas_h = (ctypes.c_double * n_al)(*qmm.AWQ_ALPHAS)
    wsa = torch.empty(qmm.awq_workspace_bytes(na, ka, ta, n_al), dtype=torch.uint8, device=dev)
    ga = ka // qmm.GROUP
    ca = torch.empty((na, ka // 2), dtype=torch.uint8, device=dev)
    sca = torch.empty((na, ga), dtype=torch.float32, device=dev)
    za = torch.empty((na, (ga + 1) // 2), dtype=torch.uint8, device=dev)
    sma = torch.empty(ka, dtype=torch.float32, device=dev)
    era = torch.empty(n_al, dtype=torch.float64, device=dev)
    ba = torch.empty(1, dtype=torch.int64, device=dev)
    cfga = f"AWQ scaling search {na}x{ka}, {ta} calibration tokens, {n_al} alphas"

    def awq(i):
        ok(lib.awq_search(P(wa), qmm.BF16, P(xa), qmm.BF16, na, ka, ta, ctypes.cast(alphas_h, ctypes.c_void_p), n_al,
                          P(ca), P(sca), P(za), P(sma), P(era), P(ba), P(wsa), wsa.numel(), S(xa)))

    # bytes: what the launches move as designed (per alpha: the weights read
    # and quantized with the factors applied on the fly, the inputs scaled to
    # bf16, the W4A16 product into fp32 and the squared error against X W^T;
    # once: the magnitudes, X W^T, the final quantization)
    fmt_a = na * ka // 2 + na * ga * 4 + na * ga // 2
    per_alpha = (2 * na * ka + fmt_a) + (2 * ta * ka + 2 * ta * ka) + (2 * ta * ka + fmt_a + 4 * ta * na) + \
        8 * ta * na
    once = 2 * ta * ka + (2 * ta * ka + 2 * na * ka + 4 * ta * na) + (2 * na * ka + fmt_a)
    ops.add(f"awq_search {na}x{ka} T={ta}", awq, n_al * per_alpha + once, "mfma",
            "awq_* kernels + i8_gemm_kernel (bf16) + quantize_g128_lds_kernel (column factors) + w4_tile_kernel",
            cfga, reads=lambda i: ["wa", "xa"], writes=lambda i: ["ca"], flops=2 * ta * na * ka * (n_al + 1),
            peak=BF16_PEAK_TFLOPS)

    # ---- 70B-class MLP decode: W4A16 B=8 then B=1, then W8A16 --------------
    for m in mats:
        for B in (1, 8):
            for use in ("w4", "w8"):
                m[f"x{B}{use}"] = workloads.activations(wl5, B, m["k"], salt=m["idx"]).to(dev)
                m[f"y{B}{use}"] = torch.empty((B, m["n"]), dtype=torch.bfloat16, device=dev)
    for B, sel in ((8, lambda i: (i + 1) % C), (1, lambda i: (i + 2) % C)):
        for m in mats:
            gemv_op(ops, lib, f"w4a16_gemv B={B} {m['n']}x{m['k']}", m["copies"], sel, m["key"], m["n"], m["k"],
                    m[f"x{B}w4"], m[f"y{B}w4"], B, qmm.BF16, cfg5, f"x{B}w4_70b{m['idx']}",
                    group="gemv_b1" if B == 1 else None)
    # weight-only INT8 on the same matrices: per-channel codes from the
    # on-device quantizer, one copy for B=1 and one for B=8
    for m in mats:
        m["q8"] = [qmm.sq_quantize_weight(m["w"]) for _ in range(2)]
    for j, B in enumerate((1, 8)):
        for m in mats:
            def w8(i, m=m, B=B, j=j):
                q, b = m["q8"][j]
                ok(lib.w8a16_gemv(P(q), P(b), m["n"], m["k"], P(m[f"x{B}w8"]), qmm.BF16, B, P(m[f"y{B}w8"]),
                                  qmm.BF16, S(q)))
            ops.add(f"w8a16_gemv B={B} {m['n']}x{m['k']}", w8,
                    m["n"] * m["k"] + m["n"] * 4 + B * m["k"] * 2 + B * m["n"] * 2, "hbm", w8_kernel_name(B, m["k"]), cfg5,
                    reads=lambda i, m=m, j=j, B=B: [f"w8_70b{m['idx']}[{j}]", f"x{B}w8_70b{m['idx']}"],
                    flops=2 * B * m["n"] * m["k"])
    for f in fmts:
        def gemv_fmt(i, f=f, m=m0):
            c, sc, z = f["copies"][(i + 1) % 2]
            ok(lib.wxa16_gemv(P(c), P(sc), P(z), m["n"], m["k"], f["group"], f["bits"], qmm._sdt(f["sdt"]), P(f["x"]),
                              qmm.BF16, 1, P(f["y"]), qmm.BF16, S(c)))
        ops.add(f"wxa16_gemv B=1 {f['tag']} {m0['n']}x{m0['k']}", gemv_fmt,
                fmt_bytes(m0["n"], m0["k"], f) + m0["k"] * 2 + m0["n"] * 2, "hbm", "gemv_fmt_kernel", cfg5,
                reads=lambda i, f=f: [f"{f['key']}[{(i + 1) % 2}]", f"x_{f['key']}"], flops=2 * m0["n"] * m0["k"])
    return ops, mats


def kernel_source(text, name):
    """The text of kernel `name` in a HIP source: from its `void name(` to the
    brace that closes its body (None if absent)."""
    i = text.find(f"void {name}(")
    if i < 0:
        return None
    j = text.find("{", text.find(")", i))
    depth = 0
    for k in range(j, len(text)):
        depth += {"{": 1, "}": -1}.get(text[k], 0)
        if depth == 0:
            return text[i:k + 1]
    return None


def gemv_traffic():
    """HBM bytes per B=1 GEMV launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the
    kernel's own source text has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_valu_kernel_traffic.json")
    try:
        rec = json.load(open(path))
        body = kernel_source(open(os.path.join(ROOT, rec["source"])).read(), rec["kernel_function"])
    except (OSError, ValueError, KeyError):
        return None
    if body is None or hashlib.sha256(body.encode()).hexdigest() != rec.get("kernel_sha256"):
        return None
    launches = list(rec["per_launch"].values())
    return round(sum(v["hbm_read_bytes"] + v["hbm_write_bytes"] for v in launches) / len(launches))


def summarize_profiles(d):
    """The per-kernel table of profiles/bench_step_all_kernels.md (printed) and
    profiles/gemv_valu_kernel_traffic.json (written) from one profiling set in
    directory d, laid out as that file's rocprofv3 commands write it: the
    kernel trace (trace/bench_results.db) and the counter runs fetch, write,
    cfetch, cwrite (the plain-copy calibration), mfma, lds and valu."""
    import collections
    import csv
    import hashlib
    import re
    import sqlite3

    def short(n):
        n = re.sub(r"^void ", "", n.replace("qmm::(anonymous namespace)::", "").replace("(anonymous namespace)::", ""))
        return re.sub(r"\(.*$", "", n)

    def rows(run):
        return list(csv.DictReader(open(os.path.join(d, run, "run_counter_collection.csv"))))

    def pmc(run):
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in rows(run):
            agg[(short(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return agg

    mean = lambda v: sum(v) / len(v)
    dur = collections.defaultdict(list)
    db = sqlite3.connect(os.path.join(d, "trace", "bench_results.db"))
    for name, grid, t in db.execute("select name, grid_x*grid_y*grid_z, duration from kernels").fetchall():
        dur[(short(name), grid)].append(t / 1e3)
    total = sum(sum(v) for v in dur.values())
    copy = 256 << 20   # --calibrate-copy's buffer
    fscale = copy / (mean([float(r["Counter_Value"]) for r in rows("cfetch") if "copyBuffer" in r["Kernel_Name"]]) * 1024)
    wscale = copy / (mean([float(r["Counter_Value"]) for r in rows("cwrite") if "copyBuffer" in r["Kernel_Name"]]) * 1024)
    F, W, Mf, L, V = pmc("fetch"), pmc("write"), pmc("mfma"), pmc("lds"), pmc("valu")
    for (k, g), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        if k.startswith("at::native") or "elementwise" in k or "distribution" in k:
            continue
        t = mean(v)
        rd, wr = F.get((k, g), {}).get("FETCH_SIZE"), W.get((k, g), {}).get("WRITE_SIZE")
        rds = f"{mean(rd) * 1024 * fscale / 2**20:.1f}" if rd else "-"
        wrs = f"{mean(wr) * 1024 * wscale / 2**20:.1f}" if wr else "-"
        m, mf = Mf.get((k, g), {}), "-"
        if m.get("SQ_VALU_MFMA_BUSY_CYCLES") and m.get("GRBM_GUI_ACTIVE"):
            busy = mean(m["SQ_VALU_MFMA_BUSY_CYCLES"]) / (mean(m["GRBM_GUI_ACTIVE"]) / 8 * 1024)
            ops = 512 * sum(mean(m.get(c, [0])) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                                                          "SQ_INSTS_VALU_MFMA_MOPS_F8"))
            if busy > 0.001:
                mf = f"{100 * busy:.1f}% ({ops / (t * 1e-6) / 1e12:.0f} T/s)"
        l, ld = L.get((k, g), {}), "-"
        if l.get("SQ_LDS_IDX_ACTIVE") and mean(l["SQ_LDS_IDX_ACTIVE"]) > 0:
            ld = f"{100 * mean(l['SQ_LDS_BANK_CONFLICT']) / mean(l['SQ_LDS_IDX_ACTIVE']):.1f}%"
        vv = V.get((k, g), {})
        va = f"{mean(vv['SQ_INSTS_VALU']) / 1e6:.2f}" if vv.get("SQ_INSTS_VALU") else "-"
        print(f"| `{k}` | {g} | {len(v)} | {t:.2f} | {min(v):.2f} | {max(v):.2f} | {100 * sum(v) / total:.1f}% | "
              f"{rds} | {wrs} | {mf} | {ld} | {va} |")
    # the headline kernel's traffic per launch, keyed to its source text
    grids = {917504: "28672x8192", 262144: "8192x28672"}
    per = collections.defaultdict(lambda: {"f": [], "w": []})
    for key, run, sc in (("f", "fetch", fscale), ("w", "write", wscale)):
        for r in rows(run):
            if "gemv_valu_kernel<2, 2, 1, 8, 4>" in r["Kernel_Name"] and int(r["Grid_Size"]) in grids:
                per[grids[int(r["Grid_Size"])]][key].append(float(r["Counter_Value"]) * 1024 * sc)
    src = "quantized_matmul_quantize_amd/csrc/w4a16.hip"
    body = kernel_source(open(os.path.join(ROOT, src)).read(), "gemv_valu_kernel")
    rec = {"kernel": "gemv_valu_kernel<bf16, bf16, B=1, R=8, KW=4>", "kernel_function": "gemv_valu_kernel",
           "source": src, "kernel_sha256": hashlib.sha256(body.encode()).hexdigest(),
           "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
           "per_launch": {k: {"hbm_read_bytes": round(mean(v["f"])), "hbm_write_bytes": round(mean(v["w"])),
                              "launches": len(v["f"])} for k, v in per.items()},
           "summary": "profiles/bench_step_all_kernels.md"}
    json.dump(rec, open(os.path.join(ROOT, "profiles", "gemv_valu_kernel_traffic.json"), "w"), indent=1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(min_seconds=(8.0, 6.0), max_reps=40):
    """The CPU oracle's B=1 product (dequantize + fp64 dot products) for both
    70B-class matrices on the host: the serial oracle, then its OpenMP build."""
    import oracle  # test infrastructure: only this baseline leg uses it

    wl5 = workloads.WORKLOADS["mlp70b"]
    cases = []
    for idx, (n, k) in enumerate(wl5.weights):
        w_cpu, _ = workloads.weight(wl5, idx)
        q, s, z = oracle.asym_quantize(w_cpu.float().numpy())
        del w_cpu
        x = workloads.activations(wl5, 1, k, salt=idx).float().numpy()
        cases.append((q, s, z, x, w4_bytes(n, k) + k * 2 + n * 2))

    def leg(parallel, budget):
        reps, elapsed, nbytes = 0, 0.0, 0
        while reps < max_reps and (elapsed < budget or reps == 0):
            for q, s, z, x, b in cases:
                t0 = time.perf_counter()
                oracle.w4a16_reference(x, q, s, z, parallel=parallel)
                elapsed += time.perf_counter() - t0
                nbytes += b
            reps += 1
        return nbytes / elapsed / 1e9, reps, elapsed

    serial, r1, e1 = leg(False, min_seconds[0])
    par, r2, e2 = leg(True, min_seconds[1])
    threads = oracle.threads(parallel=True)
    model = cpu_model()
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(par, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"plain-C oracle W4A16 B=1 reference (dequantize + fp64 product) on both 70B-class MLP "
                      f"matrices (28672x8192 and 8192x28672): OpenMP build (output rows split over {threads} "
                      f"threads, results bit-identical to the serial oracle) {r2} repetition(s) in {e2:.1f} s; "
                      f"host {model}, {nproc} CPUs available",
            "single_thread": {"value": round(serial, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"the serial oracle, {r1} repetition(s) in {e1:.1f} s"},
            "cpu_model": model, "nproc": nproc}


def vendor_gemms(dev):
    """Context, not a denominator: the ROCm BLAS libraries (through torch) on
    the INT8 and bf16 products of the same 2048x4096x4096 shape, median of 20
    after 5 warm-up calls; None where the library call is unavailable."""
    m, n, k = 2048, 4096, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    out = {}

    def median_us(fn):
        for _ in range(5):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))

    try:
        a8 = torch.randint(-128, 128, (m, k), dtype=torch.int8, device=dev, generator=g)
        b8 = torch.randint(-128, 128, (n, k), dtype=torch.int8, device=dev, generator=g)
        us = median_us(lambda: torch._int_mm(a8, b8.t()))
        out["int8_TOPS"] = round(2 * m * n * k / us / 1e6, 1)
    except Exception:   # the context figure is optional
        out["int8_TOPS"] = None
    a16 = torch.randn(m, k, device=dev, generator=g).to(torch.bfloat16)
    b16 = torch.randn(n, k, device=dev, generator=g).to(torch.bfloat16)
    us = median_us(lambda: torch.matmul(a16, b16.t()))
    out["bf16_TFLOPs"] = round(2 * m * n * k / us / 1e6, 1)
    out["shape"] = f"{m}x{n}x{k} (torch._int_mm / torch.matmul)"
    # the dense bf16 product the W4A16 GEMM replaces: 14336x4096 bf16 weights
    # (four copies, 470 MB, rotated so that each call reads them from memory)
    wd = [torch.randn(14336, 4096, device=dev, generator=g).to(torch.bfloat16) for _ in range(4)]
    dense = {}
    for mm in (16, 64, 256):
        xd = torch.randn(mm, 4096, device=dev, generator=g).to(torch.bfloat16)
        it = iter(range(1 << 30))
        dense[f"M={mm}"] = round(median_us(lambda: torch.matmul(xd, wd[next(it) % 4].t())), 2)
    out["dense_bf16_gemm_14336x4096_us"] = dense
    del wd
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB (5 times), to scale HBM byte counters")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="print the per-kernel profile table and write the GEMV traffic record from a profiling set "
                         "(no GPU used)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": nbytes, "calibrate_copy_bytes_written": nbytes,
                          "copies": 5}), flush=True)
        return
    print("bench: generating inputs and quantizing (untimed)", file=sys.stderr, flush=True)
    table, mats = build_ops(dev)
    ops = table.ops
    reuse = table.reuse_distances()
    warm = [o["name"] for o in ops if o["bound"] == "hbm" and reuse[o["name"]] < COLD_BYTES]
    if warm:
        raise SystemExit(f"bench: these HBM-bound ops would read cache-warm operands: {warm}")
    torch.cuda.synchronize()

    # Ops of a group (the two B=1 GEMVs) run back to back between one pair of
    # events: an event between two ~20 us kernels would add the next
    # kernel's dispatch latency (~2 us) to its time.  Each op of a group is
    # credited with the group's time divided by its size.
    def first_of_group(j):
        return ops[j].get("group") is None or j == 0 or ops[j - 1].get("group") != ops[j]["group"]

    def last_of_group(j):
        return ops[j].get("group") is None or j == len(ops) - 1 or ops[j + 1].get("group") != ops[j]["group"]

    def step(i, events):
        for j, op in enumerate(ops):
            if events is not None and first_of_group(j):
                events[j][0].record()
            op["fn"](i)
            if events is not None and last_of_group(j):
                events[j][1].record()

    print(f"bench: {args.warmup} warmup + {args.steps} timed steps of {len(ops)} ops", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()

    per_step_events = [[(HipEvent(), HipEvent()) for _ in ops] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i, per_step_events[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    print("bench: timed steps done", file=sys.stderr, flush=True)

    breakdown = {}
    for j, op in enumerate(ops):
        j0, j1 = j, j
        while not first_of_group(j0):
            j0 -= 1
        while not last_of_group(j1):
            j1 += 1
        size = j1 - j0 + 1
        ms = [per_step_events[i][j0][0].elapsed_time(per_step_events[i][j1][1]) / size for i in range(args.steps)]
        avg_us = 1e3 * float(np.mean(ms))
        rec = {"config": op["config"], "kernel": op["kernel"], "avg_us": round(avg_us, 3),
               "median_us": round(1e3 * float(np.median(ms)), 3),
               "p10_us": round(1e3 * float(np.percentile(ms, 10)), 3),
               "p90_us": round(1e3 * float(np.percentile(ms, 90)), 3), "alg_bytes": op["bytes"],
               "GBps": round(op["bytes"] / avg_us / 1e3, 2),
               "hbm_frac": round(op["bytes"] / avg_us / 1e3 / HBM_PEAK_GBPS, 4)}
        if op["flops"]:
            peak = op["peak"] or BF16_PEAK_TFLOPS
            rec["TFLOPs"] = round(op["flops"] / avg_us / 1e6, 2)
            rec["mfma_frac"] = round(op["flops"] / avg_us / 1e6 / peak, 4)
        rec["bound"] = op["bound"]
        rec["reuse_MB"] = round(reuse[op["name"]] / 1e6) if reuse[op["name"]] != float("inf") else None
        if size > 1:
            rec["timing"] = f"back to back with {size - 1} other launch(es), one event pair, time split evenly"
        breakdown[op["name"]] = rec

    # Context, not a denominator: the library's plain streaming read
    # (qmm_stream_read) over 1 GiB, median of 10, after the timed steps.
    lib = qmm.lib()
    big = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    xo = torch.empty(1, dtype=torch.int32, device=dev)
    rd = []
    for _ in range(12):
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        ok(lib.qmm_stream_read(P(big), big.numel(), P(xo), S(big)))
        e1.record()
        rd.append((e0, e1))
    torch.cuda.synchronize()
    plain_read = (1 << 30) / (float(np.median([a.elapsed_time(b) for a, b in rd[2:]])) * 1e-3) / 1e9
    del big
    vendor = vendor_gemms(dev)

    gemv1 = [k for k in breakdown if k.startswith("w4a16_gemv B=1 28672") or k.startswith("w4a16_gemv B=1 8192")]
    g_bytes = sum(breakdown[k]["alg_bytes"] for k in gemv1)
    g_us = sum(breakdown[k]["avg_us"] for k in gemv1)
    value = g_bytes / g_us / 1e3

    # Cross-check of the headline's cache state: the two B=1 GEMVs again,
    # back to back as in the step, each pair right after a 1 GiB read with
    # ordinary loads (torch's max reduction), which allocate in the
    # last-level cache and so evict whatever the GEMVs could find there.
    # The step's streaming kernels read with nontemporal loads, which
    # allocate little in that cache, so the bytes counted by the in-step
    # rotation do not by themselves prove it cold.
    flush_src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    head = [op for op in ops if op["name"] in gemv1]
    fl = []
    for r in range(12):
        torch.amax(flush_src)
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for op in head:
            op["fn"](args.warmup + args.steps + r)
        e1.record()
        fl.append((e0, e1))
    torch.cuda.synchronize()
    flushed_us = 1e3 * float(np.median([a.elapsed_time(b) for a, b in fl[2:]]))
    del flush_src
    after_flush = {"GBps": round(g_bytes / flushed_us / 1e3, 2),
                   "hbm_frac": round(g_bytes / flushed_us / 1e3 / HBM_PEAK_GBPS, 4),
                   "pair_us": round(flushed_us, 3),
                   "note": "both B=1 GEMVs back to back after a 1 GiB cache-allocating read, median of 10"}

    def gbps(prefixes):
        ks = [k for k in breakdown if any(k.startswith(p) for p in prefixes)]
        return round(sum(breakdown[k]["alg_bytes"] for k in ks) / sum(breakdown[k]["avg_us"] for k in ks) / 1e3, 2)

    sq = breakdown[[k for k in breakdown if k.startswith("smooth_quant_w8a8_gemm")][0]]
    i8 = breakdown[[k for k in breakdown if k.startswith("sq_int8_gemm")][0]]
    gemm = {k.split()[1]: breakdown[k] for k in breakdown if k.startswith("w4a16_gemm")}

    result = {
        "metric": "W4A16 GEMV effective GB/s & % of HBM peak; quantize GB/s; INT8 GEMM TOPS",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "70B-class MLP decode: W4A16 GEMV B=1 on INT4 group-128 28672x8192 and 8192x28672 "
                        "(bf16 activations, fp32 accumulation); the same step also runs their quantizer, "
                        "dequantizer, B=8 GEMV and W8A16 GEMV, the 512x512 fp32 and Llama-7B-like quantize + "
                        "B=1 GEMV, the 14336x4096 quantize + W4A16 GEMM at M=16/64/256 the SmoothQuant W8A8, FP8 "
                        "W8A8 and LLM.int8() 2048x4096x4096 paths and AWQ's scaling search on a 4096x4096 layer "
                        "with 2048 calibration tokens",
            "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
            "plain_read_GBps": round(plain_read, 1),
            "headline_after_flush": after_flush,
            "vendor_library_gemms": vendor,
            "quantize_GBps": gbps(["quantize 28672x8192", "quantize 8192x28672"]),
            "quantize_GBps_llama7b": gbps(["quantize 4096x4096", "quantize 11008x4096"]),
            "quantize_GBps_gemm_14336x4096": gbps(["quantize 14336x4096"]),
            "gemv_b1_GBps_llama7b": gbps(["w4a16_gemv B=1 4096x4096", "w4a16_gemv B=1 11008x4096"]),
            "format_variants_GBps": {f"{k.split()[0]} {k.split()[2]}": breakdown[k]["GBps"] for k in breakdown
                                     if k.startswith("quantize_ex") or k.startswith("wxa16_gemv")},
            "gemm_TFLOPs": {k: v.get("TFLOPs") for k, v in gemm.items()},
            "int8_gemm_TOPS": i8.get("TFLOPs"),
            "fp8_gemm_TFLOPs": breakdown[[k for k in breakdown if k.startswith("fp8_gemm")][0]].get("TFLOPs"),
            "w8a8_online_TOPS": sq.get("TFLOPs"),
            "llm_int8_TOPS": breakdown[[k for k in breakdown if k.startswith("llm_int8_gemm")][0]].get("TFLOPs"),
            "awq_search_ms": round(breakdown[[k for k in breakdown if k.startswith("awq_search")][0]]["avg_us"] / 1e3,
                                   3),
            "weight_copies_rotated_70b": COPIES_70B,
            "min_reuse_MB_hbm_ops": round(min(reuse[o["name"]] for o in ops if o["bound"] == "hbm") / 1e6),
        },
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": gemv_traffic(),
                     "alg_bytes_per_launch": round(g_bytes / len(gemv1)),
                     "kernel": "gemv_valu_kernel (w4a16_gemv B=1), both 70B-class matrices"},
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
