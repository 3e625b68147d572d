"""The roofline model the benchmark uses to call a matmul memory- or
compute-bound, checked against the decode table printed in "Quantization from
Scratch: Scale, Zero-Point, GPTQ and AWQ", "What it buys at decode" (an 8B
model on a 3.35 TB/s, 989 TFLOP/s GPU; fixture tests/golden/decode_roofline_h100.json)."""
import json
import os

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "decode_roofline_h100.json")


def test_decode_table_of_the_page():
    g = json.load(open(GOLDEN))
    p, bw, fl = g["model_params"], g["bandwidth_Bps"], g["flops"]
    int4 = g["int4_bits_per_weight"] / 8
    for row in g["rows"]:
        b16 = bench.decode_step_ms(p, row["batch"], 2.0, bw, fl)
        i4 = bench.decode_step_ms(p, row["batch"], int4, bw, fl)
        assert abs(b16 - row["bf16_ms"]) <= 0.005 + 1e-9, (row, b16)
        assert abs(i4 - row["int4_ms"]) <= 0.005 + 1e-9, (row, i4)
        assert abs(round(b16 / i4, 1) - row["speedup"]) < 1e-9, (row, b16 / i4)
    # the ridge: the largest batch whose step is still bound by the weight read
    for key, bpw in (("ridge_int4", int4), ("ridge_bf16", 2.0)):
        ridge = max(b for b in range(1, 2000) if bench.matmul_bound(b, bpw, bw, fl) == "hbm")
        assert ridge == g[key], (key, ridge)


def test_bench_bounds_on_mi355x():
    # the batched GEMM workload on MI355X (8 TB/s, 2.5 PFLOP/s bf16): 16 and
    # 64 tokens are bound by the weight read, 256 by the matrix work
    bpw = bench.w4_bytes(14336, 4096) / (14336 * 4096)
    assert [bench.matmul_bound(m, bpw) for m in (16, 64, 256)] == ["hbm", "hbm", "mfma"]
