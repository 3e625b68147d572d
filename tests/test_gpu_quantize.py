"""GPU parity: the INT4 quantizer and dequantizer against the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_quantize_amd as qmm
import workloads
from gpu_util import bits_equal, first_diff, note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def run_and_compare(w_cpu: torch.Tensor, what: str):
    note(f"quantize_groupwise {what} shape={tuple(w_cpu.shape)} dtype={w_cpu.dtype}")
    codes, scales, zeros = qmm.quantize_groupwise(w_cpu.to(DEV))
    torch.cuda.synchronize()
    rc, rs, rz = oracle.quantize_groupwise_packed(w_cpu.float().numpy())
    c, s, z = codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy()
    assert bits_equal(s, rs), f"{what} scales: {first_diff(s, rs)}"
    assert bits_equal(z, rz), f"{what} zeros: {first_diff(z, rz)}"
    assert bits_equal(c, rc), f"{what} codes: {first_diff(c, rc)}"
    return codes, scales, zeros


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", workloads.shapes_for_parity(), ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_small(dtype, shape):
    wl = workloads.WORKLOADS["mlp70b"]
    g = workloads.rng(99, shape[0] * 7 + shape[1])
    w = workloads.gaussian(g, shape, 0.02)
    workloads.plant_scale_entries(w, g, 0.01, 10.0)
    run_and_compare(workloads.to_dtype(w, dtype), f"small-{dtype}")


@pytest.mark.parametrize("name,index", [("tiny", 0), ("llama7b", 0), ("llama7b", 1), ("gemm", 0),
                                        ("smoothquant", 0), ("mlp70b", 0), ("mlp70b", 1)])
def test_quantize_full_size(name, index):
    wl = workloads.WORKLOADS[name]
    w, _ = workloads.weight(wl, index)
    run_and_compare(w, f"{name}[{index}]")


def _edge_rows():
    rows = []
    k = 1024
    six = np.array([-0.82, -0.31, 0.05, 0.27, 0.64, 1.10], np.float32)
    eight = np.array([-0.31, -0.104, 0.0, 0.052, 0.104, 0.156, 0.208, 0.47], np.float32)
    g = np.random.Generator(np.random.PCG64(5))
    r = np.zeros((16, k), np.float32)
    r[0, :128] = np.resize(six, 128)                      # worked example, tiled
    r[0, 128:256] = np.resize(eight, 128)
    r[1, :128] = 0.0                                      # all-zero group
    r[1, 128:256] = np.linspace(0.1, 0.5, 128)            # one-signed groups
    r[1, 256:384] = -np.linspace(0.1, 0.5, 128)
    r[1, 384:512] = 0.37                                  # constant group
    r[1, 512:640] = -0.37
    ties = np.array([0.0, 15.0, 2.5, 3.5, 0.5, 1.5, 4.5, 14.5], np.float32)
    r[2, :128] = np.resize(ties, 128)                     # exact ties, s = 1
    r[3] = g.standard_normal(k).astype(np.float32) * np.float32(1e-30)   # tiny scales
    r[4] = g.standard_normal(k).astype(np.float32) * np.float32(1e30)    # huge scales
    r[5] = g.standard_normal(k).astype(np.float32) * np.float32(1e-41)   # subnormal inputs
    r[6, ::2] = np.float32(1e-45)                                         # smallest subnormal
    r[7] = g.standard_normal(k).astype(np.float32)
    r[7, 5] = 1000.0                                      # one outlier
    r[8] = np.abs(g.standard_normal(k).astype(np.float32)) + np.float32(1.0)   # far from zero
    r[9] = g.integers(-7, 9, size=k).astype(np.float32)   # integer grids
    # near-ties: values placed at (j + 1/2 +- tiny) steps of a group with known range
    for row in range(10, 16):
        for grp in range(k // 128):
            s0 = np.float32(g.random() * 0.05 + 1e-3)
            z0 = int(g.integers(0, 16))
            vals = (np.arange(128) % 15 - z0 + 0.5).astype(np.float64) * s0
            vals += g.choice([-1, 0, 1], size=128) * float(s0) * 2.0 ** -22
            vals[0] = -z0 * float(s0)
            vals[1] = (15 - z0) * float(s0)
            r[row, grp * 128:(grp + 1) * 128] = vals.astype(np.float32)
    return r


def test_quantize_edge_cases_f32():
    run_and_compare(torch.from_numpy(_edge_rows()), "edge-f32")


def test_quantize_edge_cases_bf16():
    rows = _edge_rows()
    rows[4] = np.clip(rows[4], -3e38, 3e38)
    run_and_compare(workloads.to_dtype(rows, "bf16"), "edge-bf16")


def test_quantize_worked_example_codes():
    # "Quantization Explained", six-weight example, repeated to fill 128-groups.
    six = np.array([-0.82, -0.31, 0.05, 0.27, 0.64, 1.10], np.float32)
    w = np.resize(six, (4, 256)).astype(np.float32)
    codes, scales, zeros = run_and_compare(torch.from_numpy(w), "six-weights")
    assert np.allclose(scales.cpu().numpy(), 0.128, rtol=1e-6)
    z = zeros.cpu().numpy()
    assert ((z & 0xF) == 6).all() and ((z >> 4) == 6).all()


def test_quantize_deterministic():
    wl = workloads.WORKLOADS["llama7b"]
    w, _ = workloads.weight(wl, 0)
    wd = w.to(DEV)
    note("quantize_groupwise determinism 4096x4096")
    a = [t.cpu() for t in qmm.quantize_groupwise(wd)]
    b = [t.cpu() for t in qmm.quantize_groupwise(wd)]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(3, 384), (129, 2176), (512, 512)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_dequantize(dtype, shape):
    n, k = shape
    g = np.random.Generator(np.random.PCG64(n + k))
    q = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    z = g.integers(0, 16, size=(n, k // 128)).astype(np.uint8)
    s = (g.standard_normal((n, k // 128)).astype(np.float32) * np.float32(0.01))
    s = np.abs(s) + np.float32(1e-5)
    ref = oracle.asym_dequantize(q, s, z)
    codes = torch.from_numpy(oracle.pack_codes(q)).to(DEV)
    zeros = torch.from_numpy(oracle.pack_nibbles(z)).to(DEV)
    note(f"dequantize {shape} -> {dtype}")
    out = qmm.dequantize(codes, torch.from_numpy(s).to(DEV), zeros, dtype=TDT[dtype])
    got = out.cpu()
    want = torch.from_numpy(ref).to(TDT[dtype])      # one round-to-nearest-even of the oracle's fp32
    assert bits_equal(got.view(torch.uint8).numpy() if dtype != "f32" else got.numpy(),
                      want.view(torch.uint8).numpy() if dtype != "f32" else want.numpy()), dtype


@pytest.mark.parametrize("name,index", [("llama7b", 1), ("mlp70b", 0)])
def test_dequantize_full_size(name, index):
    # full-size matrices, where the dequantizer's persistent grid strides over
    # its chunks several times: the GPU's own codes (bit-exact with the
    # oracle's) dequantized to fp32 and bf16, every element bit for bit
    wl = workloads.WORKLOADS[name]
    w, _ = workloads.weight(wl, index)
    codes, scales, zeros = run_and_compare(w, f"{name}[{index}] for dequantize")
    q, s, z = oracle.asym_quantize(w.float().numpy())
    del w
    ref = oracle.asym_dequantize(q, s, z)
    for dtype in ("f32", "bf16"):
        note(f"dequantize full size {name}[{index}] -> {dtype}")
        got = qmm.dequantize(codes, scales, zeros, dtype=TDT[dtype]).cpu()
        want = torch.from_numpy(ref).to(TDT[dtype])
        if dtype == "f32":
            assert bits_equal(got.numpy(), want.numpy()), first_diff(got.numpy(), want.numpy())
        else:
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_roundtrip_error_bound():
    # Quantize on the GPU, dequantize on the GPU: |w - w_hat| <= s/2 (+ fp32 rounding).
    wl = workloads.WORKLOADS["llama7b"]
    w, _ = workloads.weight(wl, 1)
    wd = w.to(DEV)
    note("roundtrip 11008x4096")
    codes, scales, zeros = qmm.quantize_groupwise(wd)
    back = qmm.dequantize(codes, scales, zeros, dtype=torch.float32)
    err = (back - wd.float()).abs().reshape(w.shape[0], -1, 128)
    bound = scales.unsqueeze(-1) / 2 * (1 + 1e-5) + 1e-7
    assert bool((err <= bound).all())


# --------------------------------------------------------------------------
# Symmetric INT4 ("How quantization works", "The math of quantization"),
# stored in the same format with zero-point 8.
# --------------------------------------------------------------------------
def run_and_compare_sym(w_cpu: torch.Tensor, what: str):
    note(f"quantize_groupwise_symmetric {what} shape={tuple(w_cpu.shape)} dtype={w_cpu.dtype}")
    codes, scales, zeros = qmm.quantize_groupwise(w_cpu.to(DEV), symmetric=True)
    torch.cuda.synchronize()
    rc, rs, rz, _ = oracle.sym_quantize_int4_packed(w_cpu.float().numpy())
    c, s, z = codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy()
    assert bits_equal(s, rs), f"{what} scales: {first_diff(s, rs)}"
    assert bits_equal(z, rz), f"{what} zeros: {first_diff(z, rz)}"
    assert bits_equal(c, rc), f"{what} codes: {first_diff(c, rc)}"
    return codes, scales, zeros


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", workloads.shapes_for_parity(), ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_symmetric_small(dtype, shape):
    g = workloads.rng(98, shape[0] * 7 + shape[1])
    w = workloads.gaussian(g, shape, 0.02)
    workloads.plant_scale_entries(w, g, 0.01, 10.0)
    run_and_compare_sym(workloads.to_dtype(w, dtype), f"sym small-{dtype}")


def test_quantize_symmetric_edge_cases():
    # the worked examples, all-zero / one-signed / constant groups and exact
    # half-step ties, in fp32 (odd and even group counts follow from K = 1024
    # and the 3-group slice)
    rows = _edge_rows()
    w = torch.from_numpy(rows)
    run_and_compare_sym(w, "sym edge f32")
    run_and_compare_sym(w[:, :384].contiguous(), "sym edge f32, 3 groups")
    rows[4] = np.clip(rows[4], -3e38, 3e38)
    run_and_compare_sym(workloads.to_dtype(rows, "bf16"), "sym edge bf16")


@pytest.mark.parametrize("name,index", [("llama7b", 1), ("mlp70b", 0)])
def test_quantize_symmetric_full_size(name, index):
    wl = workloads.WORKLOADS[name]
    w, _ = workloads.weight(wl, index)
    run_and_compare_sym(w, f"sym {name}[{index}]")


def test_symmetric_codes_feed_the_matmuls():
    # the stored symmetric format goes through dequantize, the GEMV (B = 1, 2)
    # and the GEMM unchanged: compare with the oracle on (q + 8, s, 8)
    g = workloads.rng(97, 3)
    n, k = 300, 1152
    w = workloads.to_dtype(workloads.gaussian(g, (n, k), 0.02), "bf16")
    codes, scales, zeros = run_and_compare_sym(w, "sym for matmuls")
    _, rs, _, q = oracle.sym_quantize_int4_packed(w.float().numpy())
    qu = (q.astype(np.int16) + 8).astype(np.uint8)
    zu = np.full(rs.shape, 8, np.uint8)
    back = qmm.dequantize(codes, scales, zeros, torch.float32).cpu().numpy()
    assert bits_equal(back, oracle.asym_dequantize(qu, rs, zu, 128)), "sym dequantize"
    from gpu_util import assert_close
    for B, fn in ((1, qmm.w4a16_gemv), (2, qmm.w4a16_gemv), (33, qmm.w4a16_gemm)):
        x = workloads.to_dtype(workloads.gaussian(workloads.rng(96, B), (B, k), 1.0), "bf16")
        note(f"w4a16 on symmetric codes B={B}")
        y = fn(codes, scales, zeros, x.to(DEV), out_dtype=torch.float32).cpu()
        assert_close(y, oracle.w4a16_reference(x.float().numpy(), qu, rs, zu), f"sym codes B={B}")
