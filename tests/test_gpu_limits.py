"""GPU parity at the size limits and in degenerate shapes, in exact mode.

Every case uses integer operands in {-1, 0, 1} (epilogue terms in {-2..2}),
so the GPU result must equal the oracle's rounding of the exact sum bit for
bit.  The large cases cross the 32-bit boundaries the kernels must not wrap
at: an operand larger than 2 GiB (which the 32-bit buffer offsets of the
direct-to-LDS copies cannot address, so it takes the generic kernel; in
binary32 also on the vector lanes, whose prefetched loads use such offsets), an
output and a residual of more than 2^31 elements, and a K of a million.
Large operands repeat a seeded block of a prime number of rows, so that a
wrapped offset would read a different row.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import GUARD, Run, assert_accept, reference_block, reference_cells

pytestmark = pytest.mark.gpu


def tiled_bits(rows, cols, ld, seed, period=61, lim=1, dtype=W.F16):
    """rows x ld raw bits: a seeded ternary block of `period` rows repeated
    down the rows, NaN in the ld padding."""
    rng = np.random.default_rng(seed)
    base = W.to_bits(rng.integers(-lim, lim + 1, size=(period, cols)).astype(np.float64), dtype)
    out = np.full((rows, ld), W.NAN_BITS[dtype], dtype=base.dtype)
    reps = -(-rows // period)
    out[:, :cols] = np.tile(base, (reps, 1))[:rows]
    return out.reshape(-1)


def device_cells(run, ms, ns):
    """C at the cells (ms, ns), gathered on the device; guard bands checked there."""
    sent = run.sentinel - (1 << 32 if run.esize == 4 and run.sentinel >= 1 << 31 else 0)
    assert bool((run.Cbuf[:GUARD] == sent).all()), "write before C"
    assert bool((run.Cbuf[-GUARD:] == sent).all()), "write after C"
    idx = torch.from_numpy(GUARD + ms * run.ldc + ns).cuda()
    vals = run.Cbuf[idx].cpu().numpy()
    return vals.view(np.uint32 if run.esize == 4 else np.uint16)


def boundary_cells(M, N, ld, elem_bytes, n_random, seed):
    """Random cells plus every cell of the rows around the 2^31-byte and the
    2^31-element offsets of a [M, ld] array, and the last row."""
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, M, n_random))
    ns = list(rng.integers(0, N, n_random))
    for b in ((1 << 31) // elem_bytes, 1 << 31):
        r = b // ld
        for m in range(max(0, r - 1), min(M, r + 2)):
            for n in range(0, N, max(1, N // 64)):
                ms.append(m); ns.append(n)
    for n in range(0, N, max(1, N // 64)):
        ms.append(M - 1); ns.append(n)
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)


def test_operand_over_2gib():
    # A [66000][16392] f16 = 2.16 GB: more than the direct-to-LDS path can address
    M, N, K = 66000, 64, 16392
    assert (M - 1) * K * 2 + K * 2 > 1 << 31
    w = W.Workload("big-a", M, N, K, dtype=W.F16, out_dtype=W.F32, dist="ternary", seed=90)
    host = {"A": tiled_bits(M, K, K, seed=90), "B": tiled_bits(K, N, N, seed=91, period=K),
            "bias": None, "R": None, "scale": None}
    run = Run(w, inputs=host)
    run.launch()
    torch.cuda.synchronize()
    ms, ns = boundary_cells(M, N, K, 2, 300, seed=1)
    got = device_cells(run, ms, ns)
    ref = reference_cells(w, host, ms, ns)
    assert_accept(got, ref, W.F32, exact=True, what="A over 2 GiB")


@pytest.mark.parametrize("regtile", [None, (64, 64, 64)])
def test_f32_operand_over_2gib(regtile):
    # A [66000][8200] binary32 = 2.16 GB: past the 32-bit offsets of the direct
    # copies (matrix cores) and of the prefetched loads (vector lanes), so both
    # paths take their 64-bit addressed loads
    M, N, K = 66000, 64, 8200
    assert M * K * 4 > 1 << 31
    w = W.Workload("big-a-f32", M, N, K, dtype=W.F32, dist="ternary", seed=98, regtile=regtile)
    host = {"A": tiled_bits(M, K, K, seed=98, dtype=W.F32),
            "B": tiled_bits(K, N, N, seed=99, period=K, dtype=W.F32),
            "bias": None, "R": None, "scale": None}
    run = Run(w, inputs=host)
    run.launch()
    torch.cuda.synchronize()
    ms, ns = boundary_cells(M, N, K, 4, 300, seed=5)
    got = device_cells(run, ms, ns)
    ref = reference_cells(w, host, ms, ns)
    assert_accept(got, ref, W.F32, exact=True, what=f"binary32 A over 2 GiB, regtile={regtile}")


def test_output_and_residual_over_2g_elements():
    # C and R [46400][46400] f16 = 2.15e9 elements each; bias, ReLU, residual
    M = N = 46400
    K = 16
    assert M * N > 1 << 31
    w = W.Workload("big-c", M, N, K, dtype=W.F16, bias=True, relu=True, residual=True,
                   dist="ternary", seed=92)
    host = {"A": tiled_bits(M, K, K, seed=92), "B": tiled_bits(K, N, N, seed=93, period=K),
            "bias": tiled_bits(1, N, N, seed=94, period=1, lim=2),
            "R": tiled_bits(M, N, N, seed=95, lim=2), "scale": None}
    run = Run(w, inputs=host)
    run.launch()
    torch.cuda.synchronize()
    ms, ns = boundary_cells(M, N, N, 2, 300, seed=2)
    got = device_cells(run, ms, ns)
    ref = reference_cells(w, host, ms, ns)
    assert_accept(got, ref, W.F16, exact=True, what="C, R over 2^31 elements")


@pytest.mark.parametrize("tile", [None, (256, 256, 32), (64, 64, 64)])
def test_long_k(tile):
    # K = 2^20 + 24: a million K steps' worth of fp32 accumulation, exact
    M, N, K = 40, 72, (1 << 20) + 24
    w = W.Workload("long-k", M, N, K, dtype=W.F16, out_dtype=W.F32, dist="ternary", seed=96,
                   tile=tile)
    run = Run(w)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), W.F32, exact=True,
                  what=f"long K tile={tile}")


@pytest.mark.parametrize("shape", [(1, 1, 1), ((1 << 20) + 3, 1, 40), (1, (1 << 20) + 5, 24),
                                   (3000, 3000, 1), (17, 5, 3)])
def test_degenerate_shapes(shape):
    M, N, K = shape
    for dt in (W.F16, W.BF16, W.F32):
        w = W.Workload("degenerate", M, N, K, dtype=dt, bias=True, relu=True, residual=True,
                       dist="ternary", seed=97)
        run = Run(w)
        run.launch()
        C = run.result()
        if M * N <= 1 << 16:
            assert_accept(C, reference_block(w, run.host), dt, exact=True, what=f"{shape} {dt}")
        else:
            rng = np.random.default_rng(3)
            ms = np.concatenate([rng.integers(0, M, 2000), [0, M - 1]])
            ns = np.concatenate([rng.integers(0, N, 2000), [N - 1, 0]])
            assert_accept(C[ms, ns], reference_cells(w, run.host, ms, ns), dt, exact=True,
                          what=f"{shape} {dt}")
