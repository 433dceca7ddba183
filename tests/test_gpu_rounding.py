"""Rounding of the fp32 accumulator to a 16-bit output on every kernel
family, on sums that fall exactly halfway between neighbouring output
values: binary16 above 2048 (where the spacing is 2 or more) and in its
subnormal range (spacing 2^-24), bfloat16 above 256.  The pages fix the
accumulation in fp32 and one cast at the end ("My Triton From Scratch,
Part 16: Register Tiles", the named GEMM of "Named layouts"); the cast
rounds to nearest, ties to even.  Every input is a normal number of the
input type and every sum is exact in fp32, so the expected bits are the
oracle's round-to-nearest-even of the exact sum.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import Run, assert_accept, reference_block

pytestmark = pytest.mark.gpu

# (tile, M): the pipelined tiles, the generic kernel, the streaming tile (M <= 16)
CASES = [((256, 256, 32), 300), ((256, 192, 32), 264), ((128, 128, 32), 136),
         ((64, 64, 64), 72), ((16, 64, 256), 13)]


def _host(w, a_vals, b_vals, a_p, b_p, seed):
    rng = np.random.default_rng(seed)
    A = rng.choice(np.array(a_vals, np.float64), size=(w.M, w.K), p=a_p)
    B = rng.choice(np.array(b_vals, np.float64), size=(w.K, w.N), p=b_p)
    assert (A.astype(np.float16).astype(np.float64) == A).all()
    assert (B.astype(np.float16).astype(np.float64) == B).all()
    return {"A": A.astype(np.float16).view(np.uint16).reshape(-1),
            "B": B.astype(np.float16).view(np.uint16).reshape(-1),
            "bias": None, "R": None, "scale": None}


def _host_bf16(w, a_vals, b_vals, a_p, b_p, seed):
    # the values are small integers and powers of two: exact in bfloat16,
    # whose bits are the top half of the binary32 bits
    rng = np.random.default_rng(seed)
    A = rng.choice(np.array(a_vals, np.float32), size=(w.M, w.K), p=a_p)
    B = rng.choice(np.array(b_vals, np.float32), size=(w.K, w.N), p=b_p)
    bits = lambda X: (X.view(np.uint32) >> 16).astype(np.uint16).reshape(-1)
    assert (bits(A).astype(np.uint32) << 16 == A.view(np.uint32).reshape(-1)).all()
    return {"A": bits(A), "B": bits(B), "bias": None, "R": None, "scale": None}


@pytest.mark.parametrize("tile,M", CASES)
def test_f16_ties_above_2048(tile, M):
    # sums 2048 a + b of small integers: every odd value in [2048, 4096),
    # every value 2 mod 4 in [4096, 8192), ... is a tie
    w = W.Workload("ties", M, 320, 64, dtype=W.F16, tile=tile)
    host = _host(w, [-2048, -1, 0, 1, 2048], [-1, 0, 1],
                 [0.1, 0.2, 0.4, 0.2, 0.1], [0.25, 0.5, 0.25], seed=71)
    ref = reference_block(w, host)
    ties = np.abs(ref) > 2048
    assert ties.mean() > 0.05, "the case must contain sums past 2048"
    run = Run(w, inputs=host)
    run.launch()
    assert_accept(run.result(), ref, W.F16, exact=True, what=f"{tile} ties above 2048")


@pytest.mark.parametrize("tile,M", CASES)
def test_f16_subnormal_ties(tile, M):
    # products of (odd multiples of 2^-11) and 2^-14: odd multiples of 2^-25,
    # whose sums lie in the binary16 subnormal range, half of them on a tie
    w = W.Workload("subn", M, 320, 64, dtype=W.F16, tile=tile)
    s = 2.0 ** -11
    host = _host(w, [-3 * s, -s, 0.0, s, 3 * s], [-2.0 ** -14, 0.0, 2.0 ** -14],
                 [0.15, 0.15, 0.4, 0.15, 0.15], [0.3, 0.4, 0.3], seed=72)
    ref = reference_block(w, host)
    assert (np.abs(ref) < 2.0 ** -14).all(), "every sum subnormal in binary16"
    assert (np.abs(ref) > 0).mean() > 0.5
    run = Run(w, inputs=host)
    run.launch()
    assert_accept(run.result(), ref, W.F16, exact=True, what=f"{tile} subnormal ties")


@pytest.mark.parametrize("tile,M", CASES)
def test_bf16_ties_above_256(tile, M):
    # sums 256 a + b of small integers: every odd value in [256, 512), every
    # value 2 mod 4 in [512, 1024), ... is a tie
    w = W.Workload("tiesbf", M, 320, 64, dtype=W.BF16, tile=tile)
    host = _host_bf16(w, [-256, -1, 0, 1, 256], [-1, 0, 1],
                      [0.1, 0.2, 0.4, 0.2, 0.1], [0.25, 0.5, 0.25], seed=73)
    ref = reference_block(w, host)
    assert (np.abs(ref) > 256).mean() > 0.05, "the case must contain sums past 256"
    run = Run(w, inputs=host)
    run.launch()
    assert_accept(run.result(), ref, W.BF16, exact=True, what=f"{tile} bf16 ties above 256")
