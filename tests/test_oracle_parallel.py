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


def test_parallel_awq_search_is_bit_identical():
    # the AWQ search's products split over threads (the large parity cases
    # use it): every output bit for bit against the serial oracle
    g = np.random.Generator(np.random.PCG64(6))
    w = (g.standard_normal((40, 256)) * 0.02).astype(np.float32)
    x = g.standard_normal((33, 256)).astype(np.float32)
    x[:, 5] *= np.float32(30.0)
    for xdt in ("bf16", "f16"):
        serial = oracle.awq_search_reference(w, x, x_dtype=xdt)
        par = oracle.awq_search_reference(w, x, parallel=True, x_dtype=xdt)
        assert serial[1] == par[1]
        for a, b in zip(serial[:1] + serial[2:], par[:1] + par[2:]):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
