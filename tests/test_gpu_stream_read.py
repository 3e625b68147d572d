"""The plain streaming read used to measure bandwidth: every byte is read
once, checked by the XOR of all 32-bit words against numpy's, on sizes from
one 16-byte piece to 64 MiB with ragged tails against the kernel's stride."""
import numpy as np
import pytest
import torch

import quantized_matmul_quantize_amd as qmm
from gpu_util import note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 64 << 20])
def test_stream_read_xor(nbytes):
    g = np.random.Generator(np.random.PCG64(nbytes))
    host = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    note(f"qmm_stream_read {nbytes} bytes")
    got = qmm.stream_read(torch.from_numpy(host).to(DEV))
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert int(got.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_stream_read_rejects_ragged_bytes():
    with pytest.raises(ValueError, match="multiple of 16"):
        qmm.stream_read(torch.zeros(20, dtype=torch.uint8, device=DEV))
