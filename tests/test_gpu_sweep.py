"""A seeded random sweep over the whole call space, in exact mode.

Each case draws sizes (ragged, down to 1), storage flags, leading-dimension
padding, input and output dtypes (all nine pairs), each epilogue term on or
off, and the path: the library's own tile choice, an explicit compiled tile,
or the vector-lane register-tile GEMM with a random logical tile.  Integer
operands make every result exact, so the GPU must match the oracle's
rounding bit for bit.
"""
import numpy as np
import pytest

import thread_register_tile_amd as trt
import workloads as W
from gpu_util import Run, assert_accept, reference_block

pytestmark = pytest.mark.gpu

DTYPES = [W.F16, W.BF16, W.F32]


def draw_case(rng, i):
    M = int(rng.choice([1, 2, 7, 16, 33, 100, 257, 300, 513, 700]))
    N = int(rng.choice([1, 3, 8, 64, 65, 129, 250, 384, 600]))
    K = int(rng.choice([1, 5, 8, 31, 32, 64, 97, 256, 333]))
    opA, opB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    pad_a, pad_b = int(rng.integers(0, 10)), int(rng.integers(0, 10))
    idt, odt = int(rng.choice(DTYPES)), int(rng.choice(DTYPES))
    path = rng.choice(["auto", "tile", "regtile"])
    tile = regtile = None
    if path == "tile" and idt != W.F32:
        t = trt.tiles()[int(rng.integers(0, len(trt.tiles())))]
        tile = (t[0], t[1], t[2])
    elif path == "tile":
        tile = (128, 128, 32)
    elif path == "regtile":
        lm, ln = int(rng.integers(1, 65)), int(rng.integers(1, 65))
        mt = int(rng.choice([32, 64]))
        tm, tn = trt.regtile_thread_shape(lm, ln, mt)
        if lm // tm <= 8 and ln // tn <= 8:
            regtile = (lm, ln, mt)
    lda = (M if opA else K) + pad_a
    ldb = (K if opB else N) + pad_b
    return W.Workload(f"sweep{i}", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb, dtype=idt,
                      out_dtype=odt, bias=bool(rng.integers(0, 2)),
                      relu=bool(rng.integers(0, 2)), residual=bool(rng.integers(0, 2)),
                      row_scale=bool(rng.integers(0, 2)), dist="ternary", seed=7000 + i,
                      tile=tile, regtile=regtile)


@pytest.mark.parametrize("chunk", range(4))
def test_random_sweep_exact(chunk):
    rng = np.random.default_rng(1234 + chunk)
    for i in range(30):
        w = draw_case(rng, 100 * chunk + i)
        ldc = w.N + int(rng.integers(0, 5))
        run = Run(w, ldc=ldc)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), w.odt, exact=True,
                      what=f"case {100 * chunk + i}: {w}")
