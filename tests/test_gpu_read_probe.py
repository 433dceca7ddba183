"""GPU test of the HBM read yardstick (trt_hbm_read_probe), through the C ABI.

The probe is not part of the GEMM; it is the plain streaming read whose
bandwidth the benchmark reports as context.  Its result is pinned by a
property that holds at any size: the XOR of the per-workgroup digests equals
the XOR of all 16-byte words read, computed here with numpy.
"""
import numpy as np
import pytest
import torch

import thread_register_tile_amd as trt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    trt.lib()


@pytest.mark.parametrize("words", [1, 2047, 2048 * 256 * 4 + 5, 3_000_017])
def test_read_probe_digest(words):
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, size=(words, 4), dtype=np.uint32)
    x = torch.from_numpy(host.view(np.int32)).cuda()
    sink = trt.hbm_read_probe(x)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    exp = np.bitwise_xor.reduce(host, axis=0)
    assert np.array_equal(got, exp)


def test_read_probe_leaves_x_unchanged():
    x = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    before = x.clone()
    trt.hbm_read_probe(x)
    torch.cuda.synchronize()
    assert torch.equal(x, before)
