"""GPU parity of the register-tile GEMM on vector lanes against the oracle.

"My Triton From Scratch, Part 16: Register Tiles": any logical tile shape,
the thread shape from the deterministic policy, strided ownership, fp32
accumulators carried over K, and the fused epilogue of "Named layouts"
(section "Contract").  Exact mode (integer operands) is bit-exact; random
operands meet |C - Cref| <= 1e-2 + 1e-2 |Cref|.
"""
from dataclasses import replace

import numpy as np
import pytest

import thread_register_tile_amd as trt
import workloads as W
from gpu_util import (Run, assert_accept, assert_full_output, reference_block, reference_cells,
                      sample_cells)

pytestmark = pytest.mark.gpu

# (lm, ln, max_threads): the pages' examples under their 32-thread budget,
# non-power-of-two shapes, full 64-lane wavefronts, and tiles of more than 64
# rows (96, 256), whose K steps are loaded without prefetching
SHAPES = [(3, 17, 32), (8, 8, 32), (16, 32, 32), (1, 64, 32), (3, 17, 64), (48, 40, 64),
          (64, 64, 64), (5, 7, 64), (96, 1, 64), (24, 40, 64), (13, 7, 64), (8, 1, 1),
          (256, 2, 64)]


def rt_case(lm, ln, mt, dtype, opA, opB, pad, epi, seed, dist="ternary", odt=None):
    M, N, K = 2 * lm + 5, 2 * ln + 3, 37
    lda = (M if opA else K) + pad
    ldb = (K if opB else N) + pad
    return W.Workload("regtile-small", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb,
                      dtype=dtype, out_dtype=odt, bias=epi, relu=epi, residual=epi,
                      row_scale=epi, dist=dist, scale=1.0, seed=seed, regtile=(lm, ln, mt))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
def test_regtile_shapes_exact(shape, dtype):
    for ops in [(0, 0), (1, 0), (0, 1), (1, 1)]:
        w = rt_case(*shape, dtype, ops[0], ops[1], 3, (ops[0] + ops[1]) % 2 == 0, seed=400)
        run = Run(w, ldc=w.N + 2)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), w.odt, exact=True,
                      what=f"{shape} dt={dtype} ops={ops}")


@pytest.mark.parametrize("shape", [(3, 17, 32), (48, 40, 64), (64, 64, 64)])
@pytest.mark.parametrize("odt", [W.F16, W.BF16, W.F32])
def test_regtile_tolerance_out_dtypes(shape, odt):
    for dtype in (W.F16, W.BF16, W.F32):
        w = rt_case(*shape, dtype, 0, 0, 0, True, seed=410, dist="uniform", odt=odt)
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), odt,
                      what=f"{shape} in={dtype} out={odt}")


def test_regtile_policy_in_use():
    # the thread shape the kernel takes is the policy's; a tile whose policy
    # shape needs more than 8 registers per axis is refused
    assert trt.regtile_thread_shape(3, 17, 32) == (1, 17)
    with pytest.raises(trt.TrtError) as e:
        w = rt_case(128, 128, 64, W.F16, 0, 0, 0, False, seed=1)
        Run(w).launch()
    assert e.value.status == trt.ERR_UNSUPPORTED


def test_regtile_workload_full_size():
    # the whole output, element by element
    w = W.REGTILE
    run = Run(w)
    run.launch()
    assert_full_output(w, run.host, run.result())


def test_regtile_workload_exact_mode():
    w = replace(W.REGTILE, dist="ternary", seed=81)
    run = Run(w)
    run.launch()
    C = run.result()
    ms, ns = sample_cells(w, 400, seed=4)
    assert_accept(C[ms, ns], reference_cells(w, run.host, ms, ns), w.odt, exact=True,
                  what="regtile exact")


def test_regtile_torch_wrapper():
    import oracle
    import torch
    g = torch.Generator().manual_seed(7)
    A = torch.randint(-1, 2, (70, 45), generator=g).to(torch.bfloat16).cuda()
    B = torch.randint(-1, 2, (45, 33), generator=g).to(torch.bfloat16).cuda()
    bias = torch.randint(-2, 3, (33,), generator=g).to(torch.float32).cuda()
    C = trt.gemm_regtile(A, B, lm=3, ln=17, max_threads=32, bias=bias, relu=True,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    Ab = A.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    Bb = B.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    ref = oracle.gemm_block(70, 33, 45, Ab, 45, 0, Bb, 33, 0, W.BF16,
                            bias=bias.cpu().numpy().view(np.uint32), relu=True, out_dtype=W.F32)
    assert_accept(C.cpu().numpy().view(np.uint32), ref, W.F32, exact=True, what="wrapper")
