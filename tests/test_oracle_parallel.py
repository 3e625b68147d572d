"""The timing-only OpenMP build of the oracle (used by the benchmark's
all-cores CPU baseline) computes exactly what the serial oracle computes:
each output row is still produced by the same sequential loop."""
import numpy as np

import oracle


def test_parallel_build_is_bit_identical():
    g = np.random.Generator(np.random.PCG64(5))
    q = g.integers(0, 16, (517, 1024)).astype(np.uint8)
    s = (g.random((517, 8), dtype=np.float32) * np.float32(0.01)).astype(np.float32)
    z = g.integers(0, 16, (517, 8)).astype(np.uint8)
    for b in (1, 3):
        x = g.standard_normal((b, 1024)).astype(np.float32)
        y1 = oracle.w4a16_reference(x, q, s, z)
        yp = oracle.w4a16_reference(x, q, s, z, parallel=True)
        assert np.array_equal(y1.view(np.uint64), yp.view(np.uint64))
    w1 = oracle.asym_dequantize(q, s, z)
    wp = oracle.asym_dequantize(q, s, z, parallel=True)
    assert np.array_equal(w1.view(np.uint32), wp.view(np.uint32))
    assert oracle.threads(parallel=False) == 1 and oracle.threads(parallel=True) >= 1
