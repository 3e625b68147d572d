#!/usr/bin/env python3
"""Benchmark of the INT4 / INT8 quantized-matmul hot path on one MI355X.

One step runs every stage of the path once on synthetic, seeded inputs that
are resident in HBM before timing starts:

  70B-class MLP, bf16 weights 28672x8192 and 8192x28672 (N(0, 0.015),
  0.1% of entries x10):
    quantize_groupwise on both matrices      (group min/max, s, z, codes, packing)
    quantize_groupwise_symmetric on the first (symmetric grid, same format)
    dequantize to bf16 on both matrices
  batched W4A16 GEMM, 14336x4096 INT4 G128, X bf16 [M, 4096], M = 16, 64, 256
  SmoothQuant W8A8, X 2048x4096 (6 outlier channels x50..100), W 4096x4096:
    sq_smooth_factors, sq_quantize_weight, per-tensor activation quantization
    (the W8A8 baseline: X read twice), sq_int8_gemm alone (i8-MFMA GEMM
    and rescale to bf16 on activations quantized before timing), and
    smooth_quant_w8a8_gemm (per-token smoothing + INT8 quantization, then the
    same GEMM): config.int8_gemm_TOPS is the GEMM alone, w8a8_online_TOPS the
    whole online call
  70B-class MLP decode: w4a16_gemv B=8 then B=1 on both matrices (B=1 is the
    headline kernel), back to back, then weight-only INT8 (w8a16_gemv,
    per-channel codes from sq_quantize_weight) at B=1 and B=8 on the same
    matrices, at the end of the step

The packed weights exist in 3 copies per matrix and successive steps rotate
through them, so a kernel never finds its operands left in the 256 MB
last-level cache by the previous use (every copy is touched once per 3 steps,
with GBs of other traffic in between).

Every kernel is bracketed by events on the stream it runs on (the library
launches on torch's current stream), so per-kernel times come from the timed
steps themselves; the two B=1 GEMVs run back to back inside one event pair
(an event between them would add the second launch's dispatch latency to its
time) and share its time.  `value` is the effective bandwidth of the B=1
GEMVs: algorithmic bytes (packed codes, scales, zero-points, activations in,
outputs out) over their kernel time.  The CPU baseline times the plain C oracle's
reference product for the same GEMVs on the host.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
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
COPIES = 3


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



def w4_kernel_name(M, N, dev):
    """Which W4A16 MFMA kernel the library picks for M tokens and N weight rows
    (the rule in w4a16.hip's launchers), for labelling only."""
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

def w4_bytes(n, k):
    c, s, z = qmm.w4_sizes(n, k)
    return c + s + z


def build_ops(dev):
    """Allocate every input/output and return the ordered list of timed ops."""
    ops = []
    wl5 = workloads.WORKLOADS["mlp70b"]
    mats = []
    for idx, (n, k) in enumerate(wl5.weights):
        w_cpu, _ = workloads.weight(wl5, idx)
        w = w_cpu.to(dev)
        del w_cpu
        copies = [qmm.quantize_groupwise(w) for _ in range(COPIES)]
        what = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
        x1 = workloads.activations(wl5, 1, k, salt=idx).to(dev)
        x8 = workloads.activations(wl5, 8, k, salt=idx).to(dev)
        y1 = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
        y8 = torch.empty((8, n), dtype=torch.bfloat16, device=dev)
        mats.append(dict(n=n, k=k, w=w, copies=copies, what=what, x1=x1, x8=x8, y1=y1, y8=y8))
    wb = w4_bytes  # shorthand

    # Copy use per step i: the quantizer writes copy i%3, the dequantizer reads
    # copy (i+2)%3, the GEMVs read copy (i+1)%3 (written two steps earlier).
    for m in mats:
        n, k = m["n"], m["k"]
        lib = qmm.lib()

        def quant(i, m=m):
            c, s, z = m["copies"][i % COPIES]
            st = lib.quantize_groupwise(qmm._ptr(m["w"]), qmm.BF16, m["n"], m["k"], 128, 4, qmm._ptr(c),
                                        qmm._ptr(s), qmm._ptr(z), qmm._stream(m["w"]))
            assert st == 0, st
        ops.append(dict(name=f"quantize {n}x{k}", fn=quant, bytes=n * k * 2 + wb(n, k), flops=0, bound="hbm",
                        kernel="quantize_g128_lds_kernel"))

    # Symmetric INT4 on the first matrix, into buffers of its own (same
    # format; not part of quantize_GBps).
    m0 = mats[0]
    sym_out = qmm.quantize_groupwise(m0["w"], symmetric=True)

    def quant_sym(i, m=m0):
        c, s, z = sym_out
        st = lib.quantize_groupwise_symmetric(qmm._ptr(m["w"]), qmm.BF16, m["n"], m["k"], 128, 4, qmm._ptr(c),
                                              qmm._ptr(s), qmm._ptr(z), qmm._stream(m["w"]))
        assert st == 0, st
    ops.append(dict(name=f"quantize_symmetric {m0['n']}x{m0['k']}", fn=quant_sym,
                    bytes=m0["n"] * m0["k"] * 2 + wb(m0["n"], m0["k"]), flops=0, bound="hbm",
                    kernel="quantize_g128_lds_kernel (symmetric)"))

    for m in mats:
        n, k = m["n"], m["k"]

        def deq(i, m=m):
            c, s, z = m["copies"][(i + 2) % COPIES]
            st = qmm.lib().dequantize(qmm._ptr(c), qmm._ptr(s), qmm._ptr(z), m["n"], m["k"], 128, 4,
                                      qmm._ptr(m["what"]), qmm.BF16, qmm._stream(c))
            assert st == 0, st
        ops.append(dict(name=f"dequantize {n}x{k}", fn=deq, bytes=wb(n, k) + n * k * 2, flops=0, bound="hbm",
                        kernel="dequantize_g128_kernel"))

    # Batched GEMM.
    wl3 = workloads.WORKLOADS["gemm"]
    n3, k3 = wl3.weights[0]
    w3, _ = workloads.weight(wl3, 0)
    w3d = w3.to(dev)
    g3 = [qmm.quantize_groupwise(w3d) for _ in range(COPIES)]
    del w3d
    for M in wl3.batches:
        X = workloads.activations(wl3, M, k3).to(dev)
        Y = torch.empty((M, n3), dtype=torch.bfloat16, device=dev)

        def gemm(i, X=X, Y=Y, M=M):
            c, s, z = g3[i % COPIES]
            st = qmm.lib().w4a16_gemm(qmm._ptr(c), qmm._ptr(s), qmm._ptr(z), n3, k3, 128, qmm._ptr(X), qmm.BF16, M,
                                      qmm._ptr(Y), qmm.BF16, qmm._stream(X))
            assert st == 0, st
        bound = "mfma" if M >= 128 else "hbm"
        ops.append(dict(name=f"w4a16_gemm M={M} {n3}x{k3}", fn=gemm, bytes=wb(n3, k3) + M * k3 * 2 + M * n3 * 2,
                        flops=2 * M * n3 * k3, bound=bound, kernel=w4_kernel_name(M, n3, dev)))

    # SmoothQuant W8A8.
    wl4 = workloads.WORKLOADS["smoothquant"]
    n4, k4 = wl4.weights[0]
    m4 = wl4.batches[0]
    x4c, _ = workloads.sq_activations(wl4, m4, k4)
    w4c, _ = workloads.weight(wl4, 0)
    x4, w4 = x4c.to(dev), w4c.to(dev)
    smooth = torch.empty(k4, dtype=torch.float32, device=dev)
    cx, cw = torch.empty_like(smooth), torch.empty_like(smooth)
    qw = torch.empty((n4, k4), dtype=torch.int8, device=dev)
    wsc = torch.empty(n4, dtype=torch.float32, device=dev)
    y4 = torch.empty((m4, n4), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qmm.sq_workspace_bytes(m4, k4), dtype=torch.uint8, device=dev)
    lib = qmm.lib()

    def sq_factors(i):
        st = lib.sq_smooth_factors(qmm._ptr(x4), qmm.BF16, m4, qmm._ptr(w4), qmm.BF16, n4, k4, 0.5, qmm._ptr(cx),
                                   qmm._ptr(cw), qmm._ptr(smooth), qmm._stream(x4))
        assert st == 0, st

    def sq_weight(i):
        st = lib.sq_quantize_weight(qmm._ptr(w4), qmm.BF16, qmm._ptr(smooth), n4, k4, qmm._ptr(qw), qmm._ptr(wsc),
                                    qmm._stream(w4))
        assert st == 0, st

    def sq_online(i):
        st = lib.smooth_quant_w8a8_gemm(qmm._ptr(x4), qmm.BF16, qmm._ptr(smooth), qmm._ptr(qw), qmm._ptr(wsc), m4,
                                        n4, k4, qmm._ptr(y4), qmm.BF16, qmm._ptr(ws), ws.numel(), qmm._stream(x4))
        assert st == 0, st

    ops.append(dict(name=f"sq_smooth_factors {m4}x{k4} / {n4}x{k4}", fn=sq_factors,
                    bytes=(m4 + n4) * k4 * 2 + 3 * k4 * 4, flops=0, bound="hbm", kernel="colmax2_kernel"))
    ops.append(dict(name=f"sq_quantize_weight {n4}x{k4}", fn=sq_weight, bytes=n4 * k4 * 3 + k4 * 4 + n4 * 4,
                    flops=0, bound="hbm", kernel="rowquant8_kernel"))
    # The INT8 GEMM alone, on weights and activations quantized once here
    # (untimed; every step recomputes the same smoothing and weights).
    qx4 = torch.empty((m4, k4), dtype=torch.int8, device=dev)
    xsc4 = torch.empty(m4, dtype=torch.float32, device=dev)
    sq_factors(0)
    sq_weight(0)
    assert lib.sq_quantize_activation(qmm._ptr(x4), qmm.BF16, qmm._ptr(smooth), m4, k4, qmm._ptr(qx4),
                                      qmm._ptr(xsc4), qmm._stream(x4)) == 0

    def sq_gemm(i):
        st = lib.sq_int8_gemm(qmm._ptr(qx4), qmm._ptr(xsc4), qmm._ptr(qw), qmm._ptr(wsc), m4, n4, k4, qmm._ptr(y4),
                              qmm.BF16, qmm._stream(x4))
        assert st == 0, st

    qx4t = torch.empty((m4, k4), dtype=torch.int8, device=dev)
    xsc4t = torch.empty(m4, dtype=torch.float32, device=dev)

    def sq_act_tensor(i):
        st = lib.sq_quantize_activation_per_tensor(qmm._ptr(x4), qmm.BF16, qmm._ptr(smooth), m4, k4, qmm._ptr(qx4t),
                                                   qmm._ptr(xsc4t), qmm._stream(x4))
        assert st == 0, st

    ops.append(dict(name=f"sq_quantize_activation_per_tensor {m4}x{k4}", fn=sq_act_tensor,
                    bytes=2 * m4 * k4 * 2 + k4 * 4 + m4 * k4 + m4 * 4, flops=0, bound="hbm",
                    kernel="rowquant8_kernel x2 + tensor_scale_kernel"))
    ops.append(dict(name=f"sq_int8_gemm {m4}x{n4}x{k4}", fn=sq_gemm,
                    bytes=m4 * k4 + m4 * 4 + n4 * k4 + n4 * 4 + m4 * n4 * 2,
                    flops=2 * m4 * n4 * k4, bound="mfma", kernel="i8_gemm_kernel", peak=I8_PEAK_TOPS))
    ops.append(dict(name=f"smooth_quant_w8a8_gemm {m4}x{n4}x{k4}", fn=sq_online,
                    bytes=m4 * k4 * 2 + k4 * 4 + (m4 * k4 + m4 * 4) * 2 + n4 * k4 + n4 * 4 + m4 * n4 * 2,
                    flops=2 * m4 * n4 * k4, bound="mfma", kernel="i8_gemm_kernel + rowquant8_kernel", peak=I8_PEAK_TOPS))
    # Decode GEMVs last, back to back (B=8 then B=1), after the read-mostly
    # GEMMs: in a decode step a GEMV follows other matmuls, not the
    # dequantizer's ~0.9 GB of writes, whose write-back would overlap it.
    for B in (8, 1):
        for m in mats:
            n, k = m["n"], m["k"]

            def gemv(i, m=m, B=B):
                c, s, z = m["copies"][(i + 1) % COPIES]
                x, y = m[f"x{B}"], m[f"y{B}"]
                st = qmm.lib().w4a16_gemv(qmm._ptr(c), qmm._ptr(s), qmm._ptr(z), m["n"], m["k"], 128, qmm._ptr(x),
                                          qmm.BF16, B, qmm._ptr(y), qmm.BF16, qmm._stream(x))
                assert st == 0, st
            ops.append(dict(name=f"w4a16_gemv B={B} {n}x{k}", fn=gemv, bytes=wb(n, k) + B * k * 2 + B * n * 2,
                            flops=2 * B * n * k, bound="hbm",
                            kernel="gemv_valu_kernel" if B == 1 else w4_kernel_name(B, n, dev),
                            group="gemv_b1" if B == 1 else None))
    # Weight-only INT8 decode on the same matrices (per-channel codes from
    # the on-device quantizer), after the INT4 GEMVs.
    for B in (1, 8):
        for m in mats:
            n, k = m["n"], m["k"]
            if "q8" not in m:
                m["q8"], m["b8"] = qmm.sq_quantize_weight(m["w"])

            def w8(i, m=m, B=B):
                x, y = m[f"x{B}"], m[f"y{B}"]
                st = qmm.lib().w8a16_gemv(qmm._ptr(m["q8"]), qmm._ptr(m["b8"]), m["n"], m["k"], qmm._ptr(x),
                                          qmm.BF16, B, qmm._ptr(y), qmm.BF16, qmm._stream(x))
                assert st == 0, st
            ops.append(dict(name=f"w8a16_gemv B={B} {n}x{k}", fn=w8, bytes=n * k + n * 4 + B * k * 2 + B * n * 2,
                            flops=2 * B * n * k, bound="hbm", kernel="w8_gemv_kernel"))

    return ops, mats


def gemv_traffic():
    """HBM bytes per B=1 GEMV launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_valu_kernel_traffic.json")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    launches = list(rec["per_launch"].values())
    return round(sum(v["hbm_read_bytes"] + v["hbm_write_bytes"] for v in launches) / len(launches))


def cpu_baseline(mats, min_seconds=12.0, max_reps=40):
    """The CPU oracle's B=1 product for both 70B-class matrices, timed on the host."""
    import oracle  # test infrastructure: only this baseline leg uses it

    wl5 = workloads.WORKLOADS["mlp70b"]
    cases = []
    for idx, (n, k) in enumerate(wl5.weights):
        w_cpu, _ = workloads.weight(wl5, idx)
        q, s, z = oracle.asym_quantize(w_cpu.float().numpy())
        del w_cpu
        x = workloads.activations(wl5, 1, k, salt=idx).float().numpy()
        cases.append((q, s, z, x, w4_bytes(n, k) + k * 2 + n * 2))
    reps, elapsed, nbytes = 0, 0.0, 0
    while reps < max_reps and (elapsed < min_seconds or reps == 0):
        for q, s, z, x, b in cases:
            t0 = time.perf_counter()
            oracle.w4a16_reference(x, q, s, z)
            elapsed += time.perf_counter() - t0
            nbytes += b
        reps += 1
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"plain-C oracle W4A16 B=1 reference (dequantize + fp64 product) on both 70B-class MLP "
                      f"matrices (28672x8192 and 8192x28672), {reps} repetition(s), {elapsed:.1f} s, one thread "
                      f"of {os.cpu_count()} ({platform.processor() or platform.machine()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB (5 times), to scale HBM byte counters")
    args = ap.parse_args()
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
    ops, mats = build_ops(dev)
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

    print(f"bench: {args.warmup} warmup + {args.steps} timed steps of {len(ops)} kernels",
          file=sys.stderr, flush=True)
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
        rec = {"kernel": op["kernel"], "avg_us": round(avg_us, 3), "median_us": round(1e3 * float(np.median(ms)), 3),
               "alg_bytes": op["bytes"], "GBps": round(op["bytes"] / avg_us / 1e3, 2),
               "hbm_frac": round(op["bytes"] / avg_us / 1e3 / HBM_PEAK_GBPS, 4)}
        if op["flops"]:
            rec["TFLOPs"] = round(op["flops"] / avg_us / 1e6, 2)
            peak = op.get("peak", BF16_PEAK_TFLOPS)
            rec["mfma_frac"] = round(op["flops"] / avg_us / 1e6 / peak, 4)
        rec["bound"] = op["bound"]
        if size > 1:
            rec["timing"] = f"back to back with {size - 1} other launch(es), one event pair, time split evenly"
        breakdown[op["name"]] = rec

    gemv1 = [k for k in breakdown if k.startswith("w4a16_gemv B=1")]
    g_bytes = sum(breakdown[k]["alg_bytes"] for k in gemv1)
    g_us = sum(breakdown[k]["avg_us"] for k in gemv1)
    value = g_bytes / g_us / 1e3
    quant = [k for k in breakdown if k.startswith("quantize ")]
    q_gbps = sum(breakdown[k]["alg_bytes"] for k in quant) / sum(breakdown[k]["avg_us"] for k in quant) / 1e3
    sq = breakdown[[k for k in breakdown if k.startswith("smooth_quant_w8a8_gemm")][0]]
    i8 = breakdown[[k for k in breakdown if k.startswith("sq_int8_gemm")][0]]

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
                        "dequantizer and B=8 GEMV, the 14336x4096 W4A16 GEMM at M=16/64/256 and the "
                        "SmoothQuant W8A8 2048x4096x4096 path",
            "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
            "quantize_GBps": round(q_gbps, 2),
            "int8_gemm_TOPS": i8.get("TFLOPs"),
            "w8a8_online_TOPS": sq.get("TFLOPs"),
            "weight_copies_rotated": COPIES,
        },
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": gemv_traffic(),
                     "alg_bytes_per_launch": round(g_bytes / len(gemv1)),
                     "kernel": "gemv_valu_kernel (w4a16_gemv B=1), both matrices"},
        "breakdown": breakdown,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(mats)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
