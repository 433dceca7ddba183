"""GPU tests of the measurement yardsticks, through the C ABI.

Neither is part of the GEMM; the benchmark reports their rates as context.
trt_hbm_read_probe (a plain streaming read) is pinned by a property that holds
at any size: the XOR of the per-workgroup digests equals the XOR of all
16-byte words read, computed here with numpy.  trt_mfma_loop_probe (matrix
cores only) is pinned by recomputing every thread's sums of accumulators on
the host from the operand words and the documented fragment maps (16x16x32
for 16-bit types, 16x16x4 for binary32), with operands in {-1, 0, 1} so that
every fp32 sum is exact.  trt_clock_probe (shader cycles over real-time
ticks) is checked for what the counters must satisfy: every workgroup waits
at least the ticks asked for, the real-time counter's rate from a long probe
timed with events is steady, and the shader clock it implies lies within the
part's clock range.
"""
import numpy as np
import pytest
import torch

import thread_register_tile_amd as trt
import workloads as W
from oracle import layout_ref as L

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


def _fragment_product(r0, r1):
    """Result registers [64, 4] of one 16x16x32 instruction whose operand 0 /
    operand 1 registers are r0 / r1 ([64, 8] values)."""
    X = np.zeros((16, 32)); Y = np.zeros((32, 16))
    for l in range(64):
        for e in range(8):
            X[L.mfma16_a(l, e)] = r0[l, e]
            Y[L.mfma16_b(l, e)] = r1[l, e]
    D = X @ Y
    return np.array([[D[L.mfma16_c(l, r)] for r in range(4)] for l in range(64)])


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_mfma_loop_probe_sums(dtype):
    rng = np.random.default_rng(5 + dtype)
    vals = rng.integers(-1, 2, size=(1024, 8)).astype(np.float64)   # 1024 words of 8 values
    ops = torch.from_numpy(W.to_bits(vals, dtype).view(np.int16).reshape(-1)).cuda()
    iters = 3
    sums = trt.mfma_loop_probe(ops, iters, dtype).cpu().numpy()
    reg = lambda base, i: vals[base + 64 * i: base + 64 * i + 64]      # [64 lanes, 8]
    # operand words A[i]: words 0.. (i < 4) then 512.. ; B[j]: 256.. then 768..
    A = [reg(0, i) for i in range(4)] + [reg(512, i) for i in range(4)]
    B = [reg(256, j) for j in range(4)] + [reg(768, j) for j in range(4)]
    exp = np.zeros((64, 16))
    for q in range(64):
        exp[:, q % 16] += iters * _fragment_product(B[q % 8], A[q // 8]).sum(axis=1)
    # every wave of every workgroup holds the same sums
    got = sums.reshape(256 * 4, 64, 16)
    assert np.array_equal(got, np.broadcast_to(exp, got.shape))


def _fragment_product_f32(r0, r1):
    """Result registers [64, 4] of one 16x16x4 f32 instruction whose operand
    0 / operand 1 registers are r0 / r1 ([64] values)."""
    X = np.zeros((16, 4)); Y = np.zeros((4, 16))
    for l in range(64):
        X[L.mfma16f32_a(l)] = r0[l]
        Y[L.mfma16f32_b(l)] = r1[l]
    D = X @ Y
    return np.array([[D[L.mfma16_c(l, r)] for r in range(4)] for l in range(64)])


def test_mfma_loop_probe_sums_f32():
    rng = np.random.default_rng(9)
    vals = rng.integers(-1, 2, size=(1024, 4)).astype(np.float64)   # 1024 words of 4 values
    ops = torch.from_numpy(W.to_bits(vals, W.F32).view(np.int32).reshape(-1)).cuda()
    iters = 3
    sums = trt.mfma_loop_probe(ops, iters, W.F32).cpu().numpy()
    word = lambda base, i, e: vals[base + 64 * i: base + 64 * i + 64, e]   # [64 lanes]
    exp = np.zeros((64, 16))
    for q in range(16):
        d = (_fragment_product_f32(word(256, q % 4, q // 4), word(0, q // 4, q % 4)) +
             _fragment_product_f32(word(768, q % 4, q // 4), word(512, q // 4, q % 4)))
        exp[:, q] = iters * d.sum(axis=1)      # output q: the sum of accumulator q's registers
    got = sums.reshape(256 * 4, 64, 16)
    assert np.array_equal(got, np.broadcast_to(exp, got.shape))


def test_mfma_loop_probe_flops():
    assert trt.mfma_loop_probe_flops(1) == 1024 * 32 * 32768
    assert trt.mfma_loop_probe_flops(1, W.F32) == 1024 * 32 * 2048


def test_clock_probe_counters():
    # a long probe, timed with events: the real-time counter advances at a
    # fixed rate, so ticks / elapsed time is the same for two lengths
    s = torch.cuda.current_stream()
    rates = []
    for ticks in (200_000, 400_000):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        out = trt.clock_probe(ticks)
        e1.record(s)
        torch.cuda.synchronize()
        c = out.cpu().numpy()
        assert (c[:, 1] >= ticks).all() and (c[:, 1] < ticks + ticks // 10).all()
        assert (c[:, 0] > 0).all()
        rates.append(ticks / (e0.elapsed_time(e1) * 1e-3))
        # shader clock while it ran: within the part's range (0.1 - 3 GHz)
        ghz = np.median(c[:, 0] / c[:, 1]) * rates[-1] / 1e9
        assert 0.1 < ghz < 3.0, ghz
    assert abs(rates[0] - rates[1]) / rates[1] < 0.05, rates
