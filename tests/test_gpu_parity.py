"""GPU parity: the HIP path against the oracle, through the C ABI.

Small shapes that span several tiles and ragged tails, and every named
workload at its full size, are compared element by element.  Exact mode (operands
in {-1, 0, 1}, epilogue terms in {-2..2}) makes every fp32 partial sum exact,
so the output must equal the oracle rounded once, bit for bit.
Acceptance elsewhere: |C - Cref| <= 1e-2 + 1e-2 |Cref| per element.
"""
import numpy as np
import pytest
import torch

import oracle
import thread_register_tile_amd as trt
import workloads as W
from oracle import layout_ref as L

from gpu_util import (Run, assert_accept, assert_full_output, reference_block, reference_cells,
                      sample_cells)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    trt.lib()


# ---- the hardware fragment layout the ownership map is built on ---------------

MAPS = {16: (L.mfma16_a, L.mfma16_b, L.mfma16_c, 16, 32, 4),
        32: (L.mfma32_a, L.mfma32_b, L.mfma32_c, 32, 16, 16)}


@pytest.mark.parametrize("shape", [16, 32])
@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_mfma_probe_fragment_maps(dtype, shape):
    fa, fb, fc, n, kk, regs = MAPS[shape]
    rng = np.random.default_rng(21)
    X = rng.integers(-3, 4, (n, kk)).astype(np.float64)   # operand 0, rows x k
    Y = rng.integers(-3, 4, (kk, n)).astype(np.float64)   # operand 1, k x cols
    a = np.zeros((64, 8)); b = np.zeros((64, 8))
    for l in range(64):
        for e in range(8):
            i, k = fa(l, e); a[l, e] = X[i, k]
            k, j = fb(l, e); b[l, e] = Y[k, j]
    D = X @ Y
    exp = np.zeros((64, regs))
    for l in range(64):
        for r in range(regs):
            i, j = fc(l, r); exp[l, r] = D[i, j]
    ab = torch.from_numpy(W.to_bits(a, dtype).view(np.int16)).cuda()
    bb = torch.from_numpy(W.to_bits(b, dtype).view(np.int16)).cuda()
    c = trt.mfma_probe(ab, bb, dtype, shape).cpu().numpy()
    assert np.array_equal(c, exp)


def test_mfma_probe_one_hot():
    # a single nonzero product lands exactly where the declared maps say
    for (i, k, j) in [(0, 0, 0), (5, 17, 9), (15, 31, 15), (12, 8, 3)]:
        X = np.zeros((16, 32)); X[i, k] = 1.0
        Y = np.zeros((32, 16)); Y[k, j] = 2.0
        a = np.zeros((64, 8)); b = np.zeros((64, 8))
        for l in range(64):
            for e in range(8):
                ii, kk = L.mfma16_a(l, e); a[l, e] = X[ii, kk]
                kk, jj = L.mfma16_b(l, e); b[l, e] = Y[kk, jj]
        c = trt.mfma_probe(torch.from_numpy(W.to_bits(a, W.F16).view(np.int16)).cuda(),
                           torch.from_numpy(W.to_bits(b, W.F16).view(np.int16)).cuda()).cpu().numpy()
        nz = np.argwhere(c != 0)
        assert len(nz) == 1
        l, r = nz[0]
        assert L.mfma16_c(int(l), int(r)) == (i, j) and c[l, r] == 2.0


# ---- device layout maps == host maps (== oracle, checked on the CPU) ----------

@pytest.mark.parametrize("tile", [(16, 64, 32), (64, 64, 64), (128, 128, 64), (256, 256, 64),
                                  (256, 256, 32), (256, 192, 32), (16, 64, 256)])
def test_layout_dump_device_equals_host(tile):
    for mid in range(11):
        if trt.layout_size(mid, tile) < 0:
            continue
        hr, hc = trt.layout_dump_host(mid, tile)
        dr, dc = trt.layout_dump(mid, tile)
        torch.cuda.synchronize()
        assert np.array_equal(dr.cpu().numpy(), hr) and np.array_equal(dc.cpu().numpy(), hc)


# ---- small shapes, every compiled instance, full comparison ---------------------

TILES = [(16, 64, 32), (64, 64, 64), (128, 128, 64), (256, 256, 64), (256, 256, 32),
         (256, 192, 32)]


def small_case(tile, dtype, opA, opB, pad, epi, seed, dist="uniform"):
    BM, BN, BK = tile
    M, N, K = 2 * BM + 37, 2 * BN + 19, 3 * BK + 9
    if BM == 256:
        M, N, K = BM + 37, BN + 19, 2 * BK + 9
    if BK == 32 and BM == 256:
        # the pipelined kernel: k-contiguous operands need K % 8 == 0, rows-
        # contiguous ones M or N % 8 == 0; a partial last K step and ragged M,
        # N edges remain
        M, N, K = 2 * BM + 40, BN + 24, 5 * BK + 8
    lda = (M if opA else K) + pad
    ldb = (K if opB else N) + pad
    return W.Workload(f"small{tile}", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb,
                      dtype=dtype, bias=epi, relu=epi, residual=epi, dist=dist, scale=1.0,
                      seed=seed, tile=tile)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("pad", [0, 8, 3])   # 3: unaligned rows -> element path
def test_small_shapes_all_instances(tile, dtype, ops, pad):
    epi = (ops[0] + pad) % 2 == 0
    w = small_case(tile, dtype, ops[0], ops[1], pad, epi, seed=100 + pad)
    run = Run(w)
    run.launch()
    C = run.result()
    Cref = reference_block(w, run.host)
    assert_accept(C, Cref, dtype, what=f"{tile} {ops} pad={pad}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("ops", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_small_shapes_exact_mode(tile, ops):
    for dtype in (W.F16, W.BF16):
        w = small_case(tile, dtype, ops[0], ops[1], 8, True, seed=7, dist="ternary")
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dtype, exact=True,
                      what=f"exact {tile} {ops} dt={dtype}")


def test_brute_force_tiny_shapes():
    rng = np.random.default_rng(5)
    dims = list(range(1, 71))
    for trial in range(40):
        M, N, K = (int(rng.choice(dims)) for _ in range(3))
        opA, opB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        w = W.Workload("tiny-bf", M, N, K, opA=opA, opB=opB, dtype=W.F16,
                       dist="ternary", seed=1000 + trial, bias=bool(trial % 2),
                       residual=bool(trial % 3 == 0), relu=bool(trial % 2))
        run = Run(w, ldc=N + (trial % 5))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F16, exact=True,
                      what=f"M={M} N={N} K={K} op={opA}{opB}")


def test_pipelined_tile_ragged_shapes():
    # the direct-to-LDS kernel on many small ragged shapes: rows beyond M and
    # N, partial last K steps, all four storage combinations, both dtypes
    rng = np.random.default_rng(9)
    for trial in range(24):
        M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
        K = 8 * int(rng.integers(1, 40))
        opA, opB = trial % 2, (trial // 2) % 2
        # rows-contiguous operands take this kernel when their rows are whole
        # 16-byte runs; other shapes run the generic kernel on the same tile
        if opA and trial % 4 != 3:
            M = max(8, M - M % 8)
        if not opB and trial % 4 != 3:
            N = max(8, N - N % 8)
        dt = W.F16 if trial % 3 else W.BF16
        a_cols = M if opA else K
        b_cols = K if opB else N
        w = W.Workload("dma-bf", M, N, K, opA=opA, opB=opB,
                       lda=-(-a_cols // 8) * 8 + 8 * (trial % 2),
                       ldb=-(-b_cols // 8) * 8 + 8 * ((trial // 3) % 2),
                       dtype=dt, dist="ternary", seed=2000 + trial,
                       bias=bool(trial % 2), relu=bool(trial % 4 == 1),
                       residual=bool(trial % 3 == 0), tile=(256, 256, 32))
        run = Run(w, ldc=N + 4 * (trial % 3))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                      what=f"M={M} N={N} K={K} op={opA}{opB} dt={dt}")


def test_pipelined_192_tile_ragged_shapes():
    # the 256x192 tile (3 fragment columns per wave, integer-affine ownership)
    # on ragged shapes, all four storage combinations, both dtypes, with and
    # without the epilogue, and one tile grid wider than 192 columns by 8
    rng = np.random.default_rng(19)
    for trial in range(20):
        M = 8 * int(rng.integers(1, 90))
        N = 8 * int(rng.integers(1, 90)) if trial else 192 * 3 + 8
        K = 8 * int(rng.integers(1, 40))
        opA, opB = trial % 2, (trial // 2) % 2
        dt = W.F16 if trial % 3 else W.BF16
        a_cols = M if opA else K
        b_cols = K if opB else N
        w = W.Workload("dma192", M, N, K, opA=opA, opB=opB,
                       lda=a_cols + 8 * (trial % 2), ldb=b_cols + 8 * ((trial // 3) % 2),
                       dtype=dt, dist="ternary", seed=5000 + trial,
                       bias=bool(trial % 2), relu=bool(trial % 4 == 1),
                       residual=bool(trial % 3 == 0), row_scale=bool(trial % 5 == 2),
                       tile=(256, 192, 32))
        run = Run(w, ldc=N + 4 * (trial % 3))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                      what=f"M={M} N={N} K={K} op={opA}{opB} dt={dt}")


@pytest.mark.parametrize("tile", [(256, 256, 32), (256, 192, 32), (128, 128, 32)])
def test_pipelined_every_step_count(tile):
    # the main loop runs whole rounds of four K steps after nk mod 4 single
    # steps: every residue, with and without a partial last step, from one
    # step up; k-contiguous operands as short as 8 elements per row (copy
    # offsets below the 3 KiB descriptor bias)
    cases = [(8, 0), (32, 1), (40, 2), (64, 3), (96, 0), (104, 1), (128, 2), (136, 3),
             (160, 0), (264, 1), (288, 2)]
    for i, (K, ops) in enumerate(cases):
        opA, opB = ops & 1, ops >> 1
        M, N = tile[0] + 24, tile[1] + 40
        dt = W.F16 if i % 2 else W.BF16
        w = W.Workload("steps", M, N, K, opA=opA, opB=opB, lda=(M if opA else K),
                       ldb=(K if opB else N), dtype=dt, dist="ternary", seed=6000 + i,
                       bias=bool(i % 2), relu=bool(i % 3 == 0), residual=bool(i % 4 == 1),
                       tile=tile)
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                      what=f"{tile} K={K} op={opA}{opB} dt={dt}")


@pytest.mark.parametrize("tile", [(256, 256, 32), (256, 192, 32), (128, 128, 32)])
def test_pipelined_epilogue_cut_tiles(tile):
    # tiles cut by M and by N: with N a multiple of 4 the fast store phase
    # takes them (stores past row M or column N dropped, residual and row
    # scale there read as zero), otherwise the masked one; C has padded rows
    # and guard bands, every output dtype, every epilogue operand
    BM, BN = tile[0], tile[1]
    cases = [  # M, N, opA, opB, in dtype, out dtype, row scale
        (BM + 37, BN + 4, 0, 1, W.F16, W.F16, False),
        (2 * BM - 8, 2 * BN - 12, 1, 1, W.BF16, W.F32, True),
        (BM + 8, BN + 36, 0, 1, W.BF16, W.BF16, False),
        (BM + 1, 2 * BN - 8, 0, 0, W.F16, W.BF16, True),
        (BM + 5, BN + 6, 0, 1, W.F16, W.F16, True),          # N % 4 != 0: masked
        (3, BN + 20, 0, 1, W.BF16, W.F16, False),             # one partial tile row
    ]
    for i, (M, N, opA, opB, dt, odt, scale) in enumerate(cases):
        K = 72
        a_cols = M if opA else K
        b_cols = K if opB else N
        w = W.Workload("cut", M, N, K, opA=opA, opB=opB, lda=a_cols + 8, ldb=b_cols + 8,
                       dtype=dt, out_dtype=odt, dist="ternary", seed=6100 + i, bias=True,
                       relu=bool(i % 2), residual=True, row_scale=scale, tile=tile)
        run = Run(w, ldc=N + 4 + 4 * (i % 2))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), odt, exact=True,
                      what=f"{tile} M={M} N={N} op={opA}{opB} {dt}->{odt}")


@pytest.mark.parametrize("tile", [(256, 256, 32), (256, 192, 32), (128, 128, 32)])
def test_pipelined_residual_strides(tile):
    # residual rows that overlap (a positive ldr below N: the masked store
    # phase) or are padded (the fast one), on tiles cut by M and N
    BM, BN = tile[0], tile[1]
    for i, (M, N, ldr, dt) in enumerate([(BM + 40, BN + 8, BN - 24, W.F16),
                                         (2 * BM - 8, BN + 16, 1, W.BF16),
                                         (BM + 8, 2 * BN, 2 * BN + 12, W.BF16)]):
        K = 64
        w = W.Workload("ldr", M, N, K, lda=K + 8, ldb=N + 8, dtype=dt, dist="ternary",
                       seed=6200 + i, bias=True, relu=bool(i % 2), residual=True, ldr=ldr,
                       tile=tile)
        run = Run(w, ldc=N + 4)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                      what=f"{tile} M={M} N={N} ldr={ldr}")


def test_randomized_shapes_strides_and_epilogues():
    # a seeded sweep over what the boundary accepts: shapes from 1 to 700,
    # storage orders, padded or overlapping input and residual rows, padded C,
    # every input and output type, every epilogue operand, automatic and
    # explicit tiles (binary32 operands: automatic or 128x128x32, the only
    # tile they run on); every element compared with the oracle, bit-exact
    rng = np.random.default_rng(77)
    tiles = [None, None, (256, 256, 32), (256, 192, 32), (128, 128, 32), (64, 64, 64),
             (16, 64, 32), (128, 128, 64)]
    for i in range(80):
        M, N, K = (int(rng.integers(1, 700)) for _ in range(3))
        if rng.random() < 0.5:
            M, N, K = (8 * max(1, x // 8) for x in (M, N, K))
        opA, opB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        dt = [W.F16, W.BF16, W.F32][int(rng.integers(0, 3))]
        odt = [None, W.F16, W.BF16, W.F32][int(rng.integers(0, 4))]

        def ld(cols):  # padded, or (one case in ten) rows that overlap
            if rng.random() < 0.9:
                return cols + int(rng.choice([0, 0, 4, 8, 24]))
            return max(1, cols - int(rng.integers(1, max(2, cols))))
        lda, ldb = ld(M if opA else K), ld(K if opB else N)
        res = bool(rng.random() < 0.4)
        ldr = ld(N)
        tile = tiles[int(rng.integers(0, len(tiles)))]
        if dt == W.F32 and tile is not None:
            tile = (128, 128, 32)
        if tile == (16, 64, 32) and M > 64:
            tile = None
        w = W.Workload("sweep", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb, dtype=dt,
                       out_dtype=odt, dist="ternary", seed=9000 + i, bias=bool(rng.random() < 0.5),
                       relu=bool(rng.random() < 0.4), residual=res, ldr=ldr if res else None,
                       row_scale=bool(rng.random() < 0.3), tile=tile)
        run = Run(w, ldc=N + int(rng.choice([0, 0, 4, 8, 12])))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), w.odt, exact=True,
                      what=f"case {i}: M={M} N={N} K={K} op={opA}{opB} lda={lda} ldb={ldb} "
                           f"dt={dt} odt={w.odt} tile={tile} res={res} ldr={w.ldr_}")


@pytest.mark.parametrize("tile", [(256, 256, 32), (256, 192, 32), (128, 128, 32)])
def test_pipelined_tiles_overlapping_rows(tile):
    # rows-contiguous operands whose rows overlap in memory (a positive stride
    # below the row length: A^T with lda < M, row-major B with ldb < N) and a
    # partial last K step: the rows k >= K of that step lie inside the
    # operand, so they must not be read as if they were zero padding
    BM, BN, _ = tile
    for trial, (opA, opB, K) in enumerate([(1, 0, 5 * 32 + 8), (1, 1, 3 * 32 + 24),
                                           (0, 0, 4 * 32 + 16), (1, 0, 2 * 32 + 5)]):
        for dt in (W.F16, W.BF16):
            M, N = 2 * BM + 40, BN + 24
            lda = M - 48 if opA else K + 8
            ldb = N - 40 if not opB else K + 8
            w = W.Workload("overlap", M, N, K, opA=opA, opB=opB, lda=lda, ldb=ldb, dtype=dt,
                           dist="ternary", seed=6000 + trial, bias=bool(trial % 2),
                           relu=bool(trial % 2), residual=trial == 2, tile=tile)
            run = Run(w, ldc=N + 4)
            run.launch()
            assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                          what=f"{tile} op={opA}{opB} K={K} lda={lda} ldb={ldb} dt={dt}")


def test_tile_choice_uses_192_for_ragged():
    # 4000 x 3072: 256x256 tiles would leave 64 of 256 compute units idle;
    # the library picks 256x192 (all four storages give the same answer)
    w = W.RAGGED
    run = Run(w)
    run.launch(tile=None)
    C = run.result()
    ms, ns = sample_cells(w, 300, seed=3)
    assert_accept(C[ms, ns], reference_cells(w, run.host, ms, ns), w.dtype, what="ragged auto")


def test_streaming_tile_shapes():
    # the M <= 16 streaming kernel: every M up to 16, K and N edges, split-K
    # slices of unequal length, epilogue combinations, both dtypes
    rng = np.random.default_rng(13)
    for trial in range(30):
        M = 1 + trial % 16
        N = 4 * int(rng.integers(1, 200))
        K = 8 * int(rng.integers(1, 300))
        dt = W.F16 if trial % 3 else W.BF16
        w = W.Workload("skinny-bf", M, N, K, lda=K + 8 * (trial % 2), ldb=N + 4 * (trial % 3),
                       dtype=dt, dist="ternary", seed=3000 + trial, bias=bool(trial % 2),
                       relu=bool(trial % 4 == 1), residual=bool(trial % 3 == 0),
                       tile=(16, 64, 256))
        run = Run(w, ldc=N + (trial % 5))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dt, exact=True,
                      what=f"M={M} N={N} K={K} dt={dt}")


def test_streaming_tile_falls_back():
    # shapes the streaming kernel does not take still compute correctly on
    # the same logical tile (generic kernel)
    for M, N, K, opA, opB in [(5, 70, 30, 0, 0), (16, 64, 64, 1, 0), (16, 64, 64, 0, 1)]:
        w = W.Workload("skinny-fb", M, N, K, opA=opA, opB=opB, dtype=W.F16, dist="ternary",
                       seed=41, tile=(16, 64, 256))
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F16, exact=True,
                      what=f"fallback M={M} N={N} K={K} op={opA}{opB}")


def test_deterministic_runs():
    w = small_case((128, 128, 64), W.F16, 0, 0, 0, True, seed=3)
    run = Run(w)
    run.launch()
    c1 = run.result()
    run.launch()
    c2 = run.result()
    assert np.array_equal(c1, c2)


# ---- the named workloads ---------------------------------------------------------

def test_tiny_config_full():
    w = W.TINY
    run = Run(w)
    run.launch()
    C = run.result()
    assert_accept(C, reference_block(w, run.host), w.dtype, what="tiny")
    we = W.Workload("tiny-exact", 64, 64, 32, dtype=W.F16, dist="ternary", seed=1,
                    tile=(16, 64, 32))
    run = Run(we)
    run.launch()
    assert_accept(run.result(), reference_block(we, run.host), W.F16, exact=True)


def _full_size(w, n_block=None):
    # the whole output, element by element ("My Triton From Scratch, Part 16:
    # Register Tiles", section "Tests cover the mapping as a contract": the
    # GPU result against the matrix product, edges included)
    print(f"full-size parity: {w.name} {w.M}x{w.N}x{w.K}", flush=True)
    run = Run(w)
    run.launch()
    C = run.result()
    assert_full_output(w, run.host, C, n_block=n_block)
    return run, C


def test_square_full_size():
    _full_size(W.SQUARE)


def test_epilogue_full_size():
    _full_size(W.EPILOGUE)


def test_ragged_full_size():
    # padding of A^T and B holds NaN: any read of it would poison C
    run, C = _full_size(W.RAGGED)
    assert np.isfinite(oracle.decode(C, W.F16)).all()


def test_skinny_full_size():
    # B's columns in blocks of 4096: the oracle decodes 512 MiB of B per block
    _full_size(W.SKINNY, n_block=4096)


@pytest.mark.parametrize("name", ["square", "epilogue", "ragged"])
def test_named_workloads_exact_mode(name):
    from dataclasses import replace
    w = replace(W.CONFIGS[name], dist="ternary", seed=77)
    run = Run(w)
    run.launch()
    C = run.result()
    ms, ns = sample_cells(w, 400, seed=1)
    ref = reference_cells(w, run.host, ms, ns)
    assert_accept(C[ms, ns], ref, w.dtype, exact=True, what=f"{name} exact")


# ---- output dtypes and the row scale ---------------------------------------------
# "Named layouts" (NineToothed), section "Contract": a row scale is the axes-"m"
# broadcast operand; the output is the accumulator cast to the output dtype.

MIXED = [(W.F16, W.F32), (W.BF16, W.F32), (W.F16, W.BF16), (W.BF16, W.F16)]


@pytest.mark.parametrize("tile", TILES + [(16, 64, 256)])
@pytest.mark.parametrize("dts", MIXED)
@pytest.mark.parametrize("ops", [(0, 0), (1, 1)])
def test_out_dtypes_and_row_scale_exact(tile, dts, ops):
    from dataclasses import replace
    if tile[2] == 256:
        # the streaming tile: M <= 16, row-major operands, whole vector runs
        w = W.Workload("skinny-mixed", 13, 276, 168 + 8 * ops[0], lda=184, ldb=284,
                       dtype=dts[0], bias=True, relu=True, residual=True, dist="ternary",
                       seed=61)
    else:
        w = small_case(tile, dts[0], ops[0], ops[1], 8, True, seed=61, dist="ternary")
    w = replace(w, out_dtype=dts[1], row_scale=True, tile=tile)
    run = Run(w, ldc=w.N + 4)
    run.launch()
    assert_accept(run.result(), reference_block(w, run.host), dts[1], exact=True,
                  what=f"{tile} {dts} {ops}")


@pytest.mark.parametrize("dts", MIXED + [(W.F16, W.F16), (W.BF16, W.BF16)])
def test_row_scale_tolerance_mode(dts):
    from dataclasses import replace
    for tile in ((128, 128, 64), (256, 256, 32)):
        w = small_case(tile, dts[0], 0, 0, 0, True, seed=62)
        w = replace(w, out_dtype=dts[1], row_scale=True)
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), dts[1], what=f"{tile} {dts}")


def test_f32_output_without_epilogue():
    from dataclasses import replace
    for tile in TILES:
        w = replace(small_case(tile, W.BF16, 1, 0, 8, False, seed=63), out_dtype=W.F32)
        run = Run(w)
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F32, what=f"{tile}")


def test_pipelined_ragged_shapes_f32_out():
    from dataclasses import replace
    rng = np.random.default_rng(17)
    for trial in range(12):
        M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
        K = 8 * int(rng.integers(1, 40))
        opA, opB = trial % 2, (trial // 2) % 2
        if opA:
            M = max(8, M - M % 8)
        if not opB:
            N = max(8, N - N % 8)
        a_cols, b_cols = (M if opA else K), (K if opB else N)
        w = W.Workload("dma-f32", M, N, K, opA=opA, opB=opB, lda=-(-a_cols // 8) * 8,
                       ldb=-(-b_cols // 8) * 8, dtype=W.F16 if trial % 2 else W.BF16,
                       out_dtype=W.F32, row_scale=bool(trial % 3), dist="ternary",
                       seed=4000 + trial, bias=bool(trial % 2), relu=bool(trial % 4 == 1),
                       residual=bool(trial % 3 == 0), tile=(256, 256, 32))
        run = Run(w, ldc=N + 4 * (trial % 3))
        run.launch()
        assert_accept(run.result(), reference_block(w, run.host), W.F32, exact=True,
                      what=f"M={M} N={N} K={K} op={opA}{opB}")


def test_rowscale_workload_full_size():
    _full_size(W.ROWSCALE)


def test_rowscale_workload_exact_mode():
    from dataclasses import replace
    w = replace(W.ROWSCALE, dist="ternary", seed=78)
    run = Run(w)
    run.launch()
    C = run.result()
    ms, ns = sample_cells(w, 400, seed=2)
    assert_accept(C[ms, ns], reference_cells(w, run.host, ms, ns), W.F32, exact=True,
                  what="rowscale exact")
