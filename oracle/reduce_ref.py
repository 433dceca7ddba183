"""Block reduction oracle: plain Python / numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Shares no code with the
HIP library.

"My Triton From Scratch, Part 12: CUDA Tile Layouts", section "Output shape
is not always thread shape": a program instance loads a rank-1 block of
BLOCK consecutive elements and stores one scalar, their sum, maximum or
minimum.  Over an input of n elements the program instances cover blocks
b = 0 .. ceil(n / BLOCK) - 1; block b holds elements [b*BLOCK, min(n,
(b+1)*BLOCK)) -- the last one may be partial, its missing elements masked
off ("Masks and stores" in Part 16 of the same series).

Readings where the page is silent: the result is a binary32 value; the sum
is the exact sum of the (exactly decoded) elements rounded once; maximum
and minimum return an element of the block, NaN if any element is NaN.
"""
import math

import numpy as np

from . import F16, BF16, F32, decode, round_out

SUM, MAX, MIN = 0, 1, 2


def block_reduce(bits, dtype, n, block, op):
    """Reference out[b] (float64) for every block of the first n elements of
    the raw buffer `bits` (uint16 of F16/BF16, or uint32 of F32)."""
    if n < 1 or block < 1:
        raise ValueError("n and block must be positive")
    x = decode(np.ascontiguousarray(bits[:n]), dtype)
    nb = -(-n // block)
    out = np.empty(nb, dtype=np.float64)
    for b in range(nb):
        v = x[b * block: min(n, (b + 1) * block)]
        if op == SUM:
            out[b] = math.fsum(v) if np.isfinite(v).all() else float(np.sum(v))
        elif np.isnan(v).any():
            out[b] = np.nan
        else:
            out[b] = v.max() if op == MAX else v.min()
    return out


def expected_bits(ref):
    """The binary32 result: the reference rounded once to nearest even."""
    return round_out(ref, F32)
