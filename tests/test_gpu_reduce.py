"""GPU parity of the rank-1 block reduction against the oracle, through the C ABI.

"My Triton From Scratch, Part 12: CUDA Tile Layouts", section "Output shape is
not always thread shape": one binary32 scalar per block of BLOCK elements, the
last block masked.  Maximum and minimum must equal the oracle exactly (+0 and
-0 compare equal); sums, accumulated in binary32 in the kernel's own order,
must lie within the summation bound len * 2^-24 * sum|x| (plus the final
rounding) of the exact sum, and be bit-exact when every partial sum is an
integer below 2^24 (exact mode).
"""
import numpy as np
import pytest
import torch

import oracle
import thread_register_tile_amd as trt
import workloads as W
from oracle import reduce_ref as RR

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    trt.lib()


def _dev(bits):
    return torch.from_numpy(bits.view(np.int32 if bits.dtype == np.uint32 else np.int16)).cuda()


def run(bits, dtype, n, block, op, offset=0):
    """Reduce elements [offset, offset + n) of bits on the GPU; guard-checked."""
    x = _dev(bits)
    nb = -(-n // block)
    out = torch.full((nb + 64,), 12345.0, dtype=torch.float32, device="cuda")
    esz = 4 if dtype == W.F32 else 2
    trt.block_reduce_raw(x.data_ptr() + esz * offset, n, block, dtype, op,
                         out.data_ptr() + 4 * 32, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[:32] == 12345.0).all() and (o[32 + nb:] == 12345.0).all(), "write outside out"
    return o[32:32 + nb]


def check(got, bits, dtype, n, block, op, offset=0, exact=False):
    ref = RR.block_reduce(bits[offset:], dtype, n, block, op)
    if op != RR.SUM or exact:
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        # values equal (so +0 == -0), and for sums in exact mode the bits too
        assert np.array_equal(got[~nan], ref[~nan].astype(np.float32))
        if exact:
            assert np.array_equal(got[~nan].view(np.uint32), RR.expected_bits(ref[~nan]))
        return
    x = np.abs(oracle.decode(np.ascontiguousarray(bits[offset:offset + n]), dtype))
    nb = len(ref)
    absum = np.array([x[b * block:(b + 1) * block].sum() for b in range(nb)])
    lens = np.array([min(block, n - b * block) for b in range(nb)])
    bound = lens * 2.0 ** -24 * absum + 2.0 ** -24 * np.abs(ref)
    assert (np.abs(got.astype(np.float64) - ref) <= bound).all()


def data(n, dtype, dist="normal", seed=0):
    w = W.ReduceWorkload("t", n, 1, dtype=dtype, dist=dist, seed=seed)
    return W.make_reduce_input(w)


SHAPES = [(1, 1), (7, 3), (1000, 64), (4096 + 3, 1024), (65536 + 5, 8192), (100000, 10000),
          (300000, 65536), (5000, 7)]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("op", [RR.SUM, RR.MAX, RR.MIN])
def test_block_reduce_shapes(dtype, op):
    for i, (n, block) in enumerate(SHAPES):
        bits = data(n, dtype, seed=i)
        check(run(bits, dtype, n, block, op), bits, dtype, n, block, op)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
def test_block_reduce_exact_sums(dtype):
    for i, (n, block) in enumerate(SHAPES):
        bits = data(n, dtype, dist="ternary", seed=10 + i)
        check(run(bits, dtype, n, block, RR.SUM), bits, dtype, n, block, RR.SUM, exact=True)


@pytest.mark.parametrize("dtype", [W.F16, W.F32])
def test_block_reduce_unaligned_and_odd_blocks(dtype):
    # an x not 16-byte aligned, and blocks whose byte size is not a multiple
    # of 16, take the element path
    n = 50000
    bits = data(n + 8, dtype, dist="ternary", seed=21)
    for offset, block in [(1, 1024), (3, 999), (0, 1001), (0, 6)]:
        check(run(bits, dtype, n, block, RR.SUM, offset), bits, dtype, n, block, RR.SUM,
              offset=offset, exact=True)
        check(run(bits, dtype, n, block, RR.MAX, offset), bits, dtype, n, block, RR.MAX,
              offset=offset)


def test_block_reduce_nan_propagates():
    bits = data(4096, W.F32, seed=30)
    bits[5] = 0x7FC00000
    bits[3000] = 0x7FC00000
    for op in (RR.SUM, RR.MAX, RR.MIN):
        got = run(bits, W.F32, 4096, 1024, op)
        assert np.isnan(got[0]) and np.isnan(got[2]) and not np.isnan(got[1]) and \
            not np.isnan(got[3])


def test_block_reduce_full_workload_sampled():
    w = W.REDUCE
    bits = W.make_reduce_input(w)
    got = run(bits, w.dtype, w.n, w.block, w.op)
    rng = np.random.default_rng(1)
    for b in list(rng.integers(0, w.nblocks, 300)) + [0, w.nblocks - 1]:
        b = int(b)
        seg = np.ascontiguousarray(bits[b * w.block:(b + 1) * w.block])
        check(got[b:b + 1], seg, w.dtype, len(seg), w.block, w.op)
