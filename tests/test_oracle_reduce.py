"""Pins of the block-reduction oracle against closed forms and brute force.

"My Triton From Scratch, Part 12: CUDA Tile Layouts", section "Output shape
is not always thread shape": one scalar per rank-1 block.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import F16, BF16, F32
from oracle import reduce_ref as RR


def bits(x, dt):
    if dt == F32:
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).view(np.uint32))
    return oracle.round16(np.asarray(x, dtype=np.float64), dt)


@pytest.mark.parametrize("dt", [F16, BF16, F32])
def test_sum_of_ones_counts_the_block(dt):
    n, block = 1000, 64
    out = RR.block_reduce(bits(np.ones(n), dt), dt, n, block, RR.SUM)
    assert out.tolist() == [64.0] * 15 + [1000 - 15 * 64]


def test_sum_of_a_ramp_closed_form():
    n, block = 4096, 512
    x = np.arange(n) % 256            # exact in f16 and bf16 (integers < 256)
    for dt in (F16, BF16, F32):
        out = RR.block_reduce(bits(x, dt), dt, n, block, RR.SUM)
        assert out.tolist() == [2 * (255 * 256 // 2)] * 8


def test_max_min_of_permutations():
    rng = np.random.default_rng(3)
    n, block = 3000, 256
    x = np.concatenate([rng.permutation(256) for _ in range(-(-n // 256))])[:n] - 100.0
    for dt in (F16, BF16, F32):
        mx = RR.block_reduce(bits(x, dt), dt, n, block, RR.MAX)
        mn = RR.block_reduce(bits(x, dt), dt, n, block, RR.MIN)
        assert mx[:-1].tolist() == [155.0] * (len(mx) - 1)
        assert mn[:-1].tolist() == [-100.0] * (len(mn) - 1)
        tail = x[(len(mx) - 1) * block:]
        assert mx[-1] == tail.max() and mn[-1] == tail.min()


def test_nan_propagates_in_max_and_min_and_sum():
    x = np.array([1.0, np.nan, 3.0, 4.0, 5.0, 6.0])
    for op in (RR.SUM, RR.MAX, RR.MIN):
        out = RR.block_reduce(bits(x, F32), F32, 6, 3, op)
        assert np.isnan(out[0]) and not np.isnan(out[1])


def test_brute_force_exact_sums():
    rng = np.random.default_rng(4)
    for dt in (F16, BF16, F32):
        for n, block in [(1, 1), (7, 3), (100, 7), (513, 64)]:
            b = bits(rng.uniform(-10, 10, n), dt)
            x = oracle.decode(b, dt)
            out = RR.block_reduce(b, dt, n, block, RR.SUM)
            for k in range(len(out)):
                exact = sum(Fraction(float(v)) for v in x[k * block:(k + 1) * block])
                # fsum is correctly rounded: within half an ulp of the exact sum
                assert abs(Fraction(out[k]) - exact) <= Fraction(abs(out[k])) * Fraction(1, 2 ** 53)


def test_expected_bits_round_once():
    assert RR.expected_bits(np.array([1.0 + 2 ** -24]))[0] == np.float32(1.0).view(np.uint32)
    assert RR.expected_bits(np.array([1.0 + 3 * 2 ** -24]))[0] == \
        np.float32(1.0 + 2 ** -22).view(np.uint32)
