"""GPU parity of the GEMM on binary32 operands against the oracle.

The register-tile GEMM of "My Triton From Scratch, Part 16: Register Tiles"
computes in f32 throughout (section "What Version 16 does not optimize");
the library runs it on the f32 matrix cores with the same fused epilogue
("Named layouts", section "Contract").  Exact mode (integer operands) must be
bit-exact; random operands meet |C - Cref| <= 1e-2 + 1e-2 |Cref|.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import thread_register_tile_amd as trt
import workloads as W
from gpu_util import (Run, assert_accept, assert_full_output, reference_block, reference_cells,
                      sample_cells)

pytestmark = pytest.mark.gpu

F32_TILE = (128, 128, 32)


def f32_case(M, N, K, opA, opB, pad, epi, seed, dist="uniform", out_dtype=W.F32):
    lda = (M if opA else K) + pad
    ldb = (K if opB else N) + pad
    return W.Workload("f32-small", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb, dtype=W.F32,
                      out_dtype=out_dtype, bias=epi, relu=epi, residual=epi,
                      row_scale=epi, dist=dist, scale=1.0, seed=seed)


@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("pad", [0, 4, 3])   # 3: rows not 16-byte aligned -> element loads
def test_f32_inputs_ragged_tolerance(ops, pad):
    # several tiles, ragged M and N, a partial last K step
    w = f32_case(2 * 128 + 37, 2 * 128 + 19, 3 * 32 + 9, ops[0], ops[1], pad,
                 epi=(ops[0] + pad) % 2 == 0, seed=200 + pad)
    run = Run(w)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), W.F32, what=f"{ops} pad={pad}")


@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("odt", [W.F32, W.F16, W.BF16])
def test_f32_inputs_exact_mode(ops, odt):
    # integer operands: every partial sum is exact in f32, so C is bit-exact
    w = f32_case(128 + 45, 3 * 128 + 7, 4 * 32 + 20, ops[0], ops[1], 4, True, seed=210,
                 dist="ternary", out_dtype=odt)
    run = Run(w, ldc=w.N + 4)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), odt, exact=True,
                  what=f"{ops} out={odt}")


# M, N and K multiples of 4 with 16-byte aligned rows take the direct-to-LDS
# kernel; the shapes leave ragged tiles and (but for K = 64) a partial last
# K step, down to a single partial step.
DIRECT_SHAPES = [(2 * 128 + 36, 3 * 128 + 20, 5 * 32 + 12), (128, 128, 64), (36, 200, 4),
                 (300, 8, 100)]


@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("shape", DIRECT_SHAPES)
def test_f32_direct_copy_path_exact(ops, shape):
    M, N, K = shape
    w = f32_case(M, N, K, ops[0], ops[1], 8 if ops[0] == ops[1] else 0, True,
                 seed=230 + M % 7, dist="ternary")
    run = Run(w, ldc=w.N + 4)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), W.F32, exact=True,
                  what=f"{ops} {shape}")


@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_f32_direct_copy_path_tolerance(ops):
    w = f32_case(3 * 128 + 4, 2 * 128 + 60, 7 * 32 + 28, ops[0], ops[1], 4, False, seed=240)
    run = Run(w)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), W.F32, what=f"{ops}")


@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_f32_kernels_agree_bit_for_bit(ops):
    # the same values with 16-byte aligned rows (direct copies) and with
    # rows padded by one element (register-staged copies): both kernels run
    # the same products in the same order
    M, N, K = 2 * 128 + 36, 128 + 92, 3 * 32 + 20
    out = []
    for pad in (4, 1):
        w = f32_case(M, N, K, ops[0], ops[1], pad, True, seed=250)
        run = Run(w)
        run.launch()
        out.append(run.result())
    assert np.array_equal(out[0], out[1]), f"{ops}: the two binary32 kernels differ"
    ref = reference_block(w, run.host)
    assert_accept(out[0], ref, W.F32, what=f"{ops}")


def test_f32_inputs_random_shapes_exact():
    rng = np.random.default_rng(23)
    for trial in range(16):
        M, N = int(rng.integers(1, 400)), int(rng.integers(1, 400))
        K = int(rng.integers(1, 200))
        opA, opB = trial % 2, (trial // 2) % 2
        w = f32_case(M, N, K, opA, opB, int(rng.integers(0, 6)), bool(trial % 3), seed=300 + trial,
                     dist="ternary")
        run = Run(w, ldc=N + trial % 5)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F32, exact=True,
                      what=f"M={M} N={N} K={K} op={opA}{opB}")


def test_f32_inputs_explicit_tile():
    w = replace(f32_case(130, 70, 40, 0, 0, 0, False, seed=220), tile=F32_TILE)
    run = Run(w)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), W.F32, what="explicit tile")


def test_f32_binding_with_torch_tensors():
    import torch
    g = torch.Generator().manual_seed(5)
    A = torch.randn(300, 200, generator=g).cuda()
    B = torch.randn(200, 150, generator=g).cuda()
    bias = torch.randn(150, generator=g).cuda()
    C = trt.gemm(A, B, bias=bias, relu=True)
    assert C.dtype == torch.float32
    torch.cuda.synchronize()
    Ab = A.cpu().numpy().view(np.uint32).reshape(-1)
    Bb = B.cpu().numpy().view(np.uint32).reshape(-1)
    ref = oracle.gemm_block(300, 150, 200, Ab, 200, 0, Bb, 150, 0, W.F32,
                            bias=bias.cpu().numpy().view(np.uint32), relu=True, out_dtype=W.F32)
    assert_accept(C.cpu().numpy().view(np.uint32), ref, W.F32, what="binding")


def test_f32square_full_size():
    # the whole output, element by element
    w = W.F32SQUARE
    run = Run(w)
    run.launch()
    assert_full_output(w, run.host, run.result())


def test_f32_overlapping_rows():
    # rows-contiguous binary32 operands whose rows overlap (lda < M, ldb < N)
    # with a partial last K step: the direct-copy kernel's zero rows past the
    # operand's end do not exist there, so such strides take the other kernel
    for trial, (opA, opB, K) in enumerate([(1, 0, 100), (1, 1, 36), (0, 0, 68)]):
        M, N = 300, 260
        lda = M - 44 if opA else K + 4
        ldb = N - 36 if not opB else K + 4
        w = replace(f32_case(M, N, K, opA, opB, 0, bool(trial % 2), seed=700 + trial,
                             dist="ternary"), lda=lda, ldb=ldb)
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F32, exact=True,
                      what=f"op={opA}{opB} K={K} lda={lda} ldb={ldb}")


def test_f32square_exact_mode():
    w = replace(W.F32SQUARE, dist="ternary", seed=79)
    run = Run(w)
    run.launch()
    C = run.result()
    ms, ns = sample_cells(w, 400, seed=3)
    assert_accept(C[ms, ns], reference_cells(w, run.host, ms, ns), W.F32, exact=True,
                  what="f32square exact")
