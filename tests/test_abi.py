"""CPU tests of the C ABI: exports, host-side validation, host layout maps.

No compute call reaches the GPU here: trt_validate, trt_layout_dump_host,
trt_layout_rank and the error paths of trt_gemm all return before any HIP
call.  The layout maps of the library are compared element by element with
the layout oracle.
"""
import os
import re

import numpy as np
import pytest

import thread_register_tile_amd as trt
from oracle import layout_ref as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "trt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(trt_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "trt_gemm" in names and "trt_validate" in names and len(names) >= 12
    lib = trt.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    hdr = open(os.path.join(ROOT, "include", "trt.h")).read()
    v = int(re.search(r"#define TRT_ABI_VERSION (\d+)", hdr).group(1))
    assert trt.abi_version() == v


# ---- validation (NineToothed "Named layouts", "Runtime and compilation") ---------

BASE = 1 << 20     # fake, well-separated 256-byte aligned addresses: never dereferenced


def args(**kw):
    a = dict(M=64, N=64, K=32, A=BASE, lda=32, opA=0, B=BASE * 2, ldb=64, opB=0,
             C=BASE * 3, ldc=64, in_dtype=trt.F16, out_dtype=trt.F16)
    a.update(kw)
    return a


def status(tile=None, bias=0, relu=False, residual=0, ldr=0, scale=0, **kw):
    a = args(**kw)
    return trt.validate_raw(a["M"], a["N"], a["K"], a["A"], a["lda"], a["opA"], a["B"],
                            a["ldb"], a["opB"], a["C"], a["ldc"], a["in_dtype"],
                            a["out_dtype"], bias=bias, relu=relu, residual=residual,
                            ldr=ldr, scale=scale, tile=tile)


def test_valid_call():
    assert status() == trt.OK
    assert status(bias=BASE * 4, relu=True, residual=BASE * 5, ldr=64) == trt.OK
    assert status(opA=1, lda=64, opB=1, ldb=32) == trt.OK
    assert status(tile=(16, 64, 32)) == trt.OK


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), trt.ERR_SIZE), (dict(N=-1), trt.ERR_SIZE), (dict(K=0), trt.ERR_SIZE),
    (dict(M=1 << 31), trt.ERR_SIZE),
    (dict(lda=0), trt.ERR_STRIDE), (dict(ldb=-5), trt.ERR_STRIDE),
    (dict(ldc=63), trt.ERR_STRIDE),
    (dict(A=0), trt.ERR_NULL), (dict(B=0), trt.ERR_NULL), (dict(C=0), trt.ERR_NULL),
    (dict(A=BASE + 1), trt.ERR_ALIGN), (dict(C=BASE * 3 + 1), trt.ERR_ALIGN),
    (dict(in_dtype=4, out_dtype=3), trt.ERR_DTYPE),
    (dict(in_dtype=0, out_dtype=trt.F16), trt.ERR_DTYPE),
    (dict(opA=2), trt.ERR_ARG), (dict(opB=-1), trt.ERR_ARG),
    # C overlapping an input: any byte in common is an error
    (dict(C=BASE + 64 * 2), trt.ERR_OVERLAP),
    (dict(C=BASE * 2 - 2), trt.ERR_OVERLAP),
])
def test_rejections(kw, code):
    assert status(**kw) == code
    assert trt.last_error() != ""


def test_overlap_boundaries_are_exact():
    # A spans [BASE, BASE + 2*(63*32 + 32)) = [BASE, BASE + 4096)
    assert status(C=BASE + 4096) == trt.OK
    assert status(C=BASE + 4094) == trt.ERR_OVERLAP
    # C spans 2*(63*ldc + 64) bytes; ending exactly at A's start is fine
    c_bytes = 2 * (63 * 64 + 64)
    assert status(C=BASE - c_bytes) == trt.OK
    assert status(C=BASE - c_bytes + 2) == trt.ERR_OVERLAP
    # transposed A spans (K-1)*lda + M elements
    assert status(opA=1, lda=64, C=BASE + 2 * (31 * 64 + 64)) == trt.OK
    assert status(opA=1, lda=64, C=BASE + 2 * (31 * 64 + 64) - 2) == trt.ERR_OVERLAP


def test_in_place_residual_rejected():
    assert status(residual=BASE * 3, ldr=64) == trt.ERR_OVERLAP
    assert status(bias=BASE * 3 + 2) == trt.ERR_OVERLAP
    assert status(residual=BASE * 5, ldr=0) == trt.ERR_STRIDE


def test_overlapping_input_rows_are_legal():
    # lda smaller than the row: rows overlap, which is fine for inputs
    assert status(lda=1) == trt.OK


def test_workgroup_count_limit():
    # a 2^30 x 2^30 output is 2^44 tiles of 256x256: more than one launch holds
    big = 1 << 30
    assert status(M=big, N=big, ldc=big, C=1 << 40) == trt.ERR_SIZE
    assert status(M=big, N=64, ldc=64, C=1 << 40) == trt.OK


def test_unknown_tile_rejected():
    assert status(tile=(48, 64, 32)) == trt.ERR_UNSUPPORTED


def test_gemm_errors_return_before_device_work():
    # invalid calls never reach HIP, so they are safe without a GPU
    with pytest.raises(trt.TrtError) as e:
        trt.gemm_raw(0, 64, 32, BASE, 32, 0, BASE * 2, 64, 0, BASE * 3, 64, trt.F16, trt.F16)
    assert e.value.status == trt.ERR_SIZE
    with pytest.raises(trt.TrtError) as e:
        trt.gemm_raw(64, 64, 32, BASE, 32, 0, BASE * 2, 64, 0, BASE, 64, trt.F16, trt.F16)
    assert e.value.status == trt.ERR_OVERLAP


# ---- tiles and layout maps --------------------------------------------------------

def tile_configs():
    return [(bm, bn, bk, wm, wn, fr) for bm, bn, bk, wm, wn, _, fr in trt.tiles()]


def test_tile_table():
    tiles = trt.tiles()
    assert (16, 64, 32, 1, 1, 16, 16) in tiles      # the named GEMM's tile, one wave
    for bm, bn, bk, wm, wn, regs, fr in tiles:
        kl = L.kernel_layout((bm, bn), (wm, 64 * wn))
        assert kl["threads_per_block"] <= 1024
        assert regs * 64 * wm * wn == bm * bn
        assert fr in (16, 32)
        if bk != 256:   # the streaming tile owns reduced outputs, not fragments
            assert regs % (fr * fr // 64) == 0


ALL_TILES = [(16, 64, 32, 1, 1, 16), (64, 64, 64, 2, 2, 16), (128, 128, 64, 2, 2, 16),
             (256, 256, 64, 2, 2, 16), (256, 256, 32, 2, 4, 16), (256, 192, 32, 2, 2, 16),
             (128, 128, 32, 2, 2, 16), (16, 64, 256, 8, 1, 16)]
NON_GF2 = (256, 192, 32, 2, 2, 16)   # 6 fragment columns per wave: affine ownership
SKINNY = (16, 64, 256, 8, 1, 16)


def test_all_tiles_listed():
    assert sorted(tile_configs()) == sorted(ALL_TILES)


@pytest.mark.parametrize("cfg", ALL_TILES)
def test_c_owner_matches_oracle(cfg):
    assert cfg in tile_configs()
    tile = cfg[:3]
    rows, cols = trt.layout_dump_host(trt.MAP_C_OWNER, tile)
    regs = 2 if cfg == SKINNY else L.gemm_regs_per_lane(cfg)
    owner = (lambda r, l, w: L.skinny_c_owner(r, l, w)) if cfg == SKINNY else \
        (lambda r, l, w: L.gemm_c_owner(cfg, r, l, w))
    x = np.arange(rows.size)
    reg, lane, wave = x % regs, (x // regs) % 64, x // (regs * 64)
    exp = np.array([owner(int(r), int(l), int(w))
                    for r, l, w in zip(reg, lane, wave)], dtype=np.int32)
    assert np.array_equal(rows, exp[:, 0]) and np.array_equal(cols, exp[:, 1])
    # exactly once over the tile
    assert len(set(zip(rows.tolist(), cols.tolist()))) == cfg[0] * cfg[1]
    if cfg == NON_GF2:
        with pytest.raises(trt.TrtError) as e:
            trt.layout_rank(tile)
        assert e.value.status == trt.ERR_UNSUPPORTED
    else:
        rank, ib, ob = trt.layout_rank(tile)
        assert rank == ib == ob == L.log2_exact(cfg[0] * cfg[1])


# the compiled power-of-two tiles with cooperative copy maps, with their wave
# grids: (BM, BN, BK, waves along m, waves along n)
@pytest.mark.parametrize("cfg", [(16, 64, 32, 1, 1), (64, 64, 64, 2, 2), (128, 128, 64, 2, 2),
                                 (256, 256, 64, 2, 2), (256, 256, 32, 2, 4),
                                 (128, 128, 32, 2, 2)])
def test_lds_and_copy_maps_match_oracle(cfg):
    BM, BN, BK, WM, WN = cfg
    tile, G, T = cfg[:3], BK // 8, 64 * WM * WN
    # the wave grid is the compiled tile's
    assert [t[3:5] for t in trt.tiles() if t[:3] == tile] == [(WM, WN)]
    for mid, R in [(trt.MAP_LDS_SLOT_A, BM), (trt.MAP_LDS_SLOT_B, BN)]:
        slot, _ = trt.layout_dump_host(mid, tile)
        exp = [L.lds_slot(r, g, G) for r in range(R) for g in range(G)]
        assert slot.tolist() == exp
    for mid, R, fn in [(trt.MAP_COPY_KCONTIG_A, BM, L.copy_kcontig),
                       (trt.MAP_COPY_KCONTIG_B, BN, L.copy_kcontig),
                       (trt.MAP_COPY_MNCONTIG_A, BM, L.copy_mncontig),
                       (trt.MAP_COPY_MNCONTIG_B, BN, L.copy_mncontig)]:
        r, c = trt.layout_dump_host(mid, tile)
        n = r.size
        exp = [fn(R, G, T, x % T, x // T) or (-1, -1) for x in range(n)]
        assert list(zip(r.tolist(), c.tolist())) == [tuple(e) for e in exp]


def test_layout_dump_host_errors():
    with pytest.raises(trt.TrtError):
        trt.layout_dump_host(99, (16, 64, 32))
    assert trt.layout_size(trt.MAP_C_OWNER, (48, 64, 32)) == -1


@pytest.mark.parametrize("tile", [(256, 256, 32), (256, 192, 32)])
def test_dma_slot_maps_match_oracle(tile):
    for mid, R in [(trt.MAP_DMA_KC_SLOT_A, tile[0]), (trt.MAP_DMA_KC_SLOT_B, tile[1])]:
        slot, _ = trt.layout_dump_host(mid, tile)
        assert slot.tolist() == [L.dma_kc_slot(r, g) for r in range(R) for g in range(4)]
    for mid, R in [(trt.MAP_DMA_MN_SLOT_A, tile[0]), (trt.MAP_DMA_MN_SLOT_B, tile[1])]:
        slot, _ = trt.layout_dump_host(mid, tile)
        assert slot.tolist() == [L.dma_mn_slot(R, k, c) for k in range(32) for c in range(R // 8)]

    # not defined for tiles without the 32-wide K step
    assert trt.layout_size(trt.MAP_DMA_KC_SLOT_A, (256, 256, 64)) == -1
    # the 256x192 tile has no generic-kernel copy maps
    assert all(trt.layout_size(m, (256, 192, 32)) == -1 for m in range(1, 7))
    # the streaming tile has only its ownership map
    assert trt.layout_size(trt.MAP_C_OWNER, (16, 64, 256)) == 1024
    assert all(trt.layout_size(m, (16, 64, 256)) == -1 for m in range(1, 11))


# ---- the HBM read yardstick: argument checks (no HIP call on error) ---------------

@pytest.mark.parametrize("kw,code", [
    (dict(x=0), trt.ERR_NULL), (dict(sink=0), trt.ERR_NULL),
    (dict(nbytes=0), trt.ERR_SIZE), (dict(nbytes=24), trt.ERR_SIZE),
    (dict(sink_bytes=trt.READ_PROBE_SINK_BYTES - 16), trt.ERR_SIZE),
    (dict(x=BASE + 8), trt.ERR_ALIGN), (dict(sink=BASE * 2 + 4), trt.ERR_ALIGN),
    (dict(sink=BASE + 4096), trt.ERR_OVERLAP),
    (dict(sink=BASE - trt.READ_PROBE_SINK_BYTES + 16), trt.ERR_OVERLAP),
])
def test_read_probe_rejections(kw, code):
    a = dict(x=BASE, nbytes=1 << 16, sink=BASE * 2, sink_bytes=trt.READ_PROBE_SINK_BYTES)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.hbm_read_probe_raw(a["x"], a["nbytes"], a["sink"], a["sink_bytes"])
    assert e.value.status == code
    assert trt.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(ops=0), trt.ERR_NULL), (dict(sink=0), trt.ERR_NULL),
    (dict(dtype=4), trt.ERR_DTYPE), (dict(iters=0), trt.ERR_ARG),
    (dict(sink_bytes=trt.MFMA_PROBE_SINK_BYTES - 64), trt.ERR_SIZE),
    (dict(ops=BASE + 8), trt.ERR_ALIGN), (dict(sink=BASE * 8 + 32), trt.ERR_ALIGN),
    (dict(sink=BASE + 4096), trt.ERR_OVERLAP),
])
def test_mfma_probe_rejections(kw, code):
    a = dict(dtype=trt.F16, ops=BASE, iters=4, sink=BASE * 8,
             sink_bytes=trt.MFMA_PROBE_SINK_BYTES)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.mfma_loop_probe_raw(a["dtype"], a["ops"], a["iters"], a["sink"], a["sink_bytes"])
    assert e.value.status == code


@pytest.mark.parametrize("kw,code", [
    (dict(sink=0), trt.ERR_NULL), (dict(ticks=0), trt.ERR_ARG),
    (dict(ticks=(1 << 27) + 1), trt.ERR_ARG),
    (dict(sink_bytes=trt.CLOCK_PROBE_SINK_BYTES - 8), trt.ERR_SIZE),
    (dict(sink=BASE + 4), trt.ERR_ALIGN),
])
def test_clock_probe_rejections(kw, code):
    a = dict(ticks=100, sink=BASE, sink_bytes=trt.CLOCK_PROBE_SINK_BYTES)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.clock_probe_raw(a["ticks"], a["sink"], a["sink_bytes"])
    assert e.value.status == code


# ---- output dtypes and the row scale ----------------------------------------------

def test_epilogue_struct_layout():
    import ctypes
    # include/trt.h: bias, relu, residual, ldr, row_scale (row_scale appended)
    assert ctypes.sizeof(trt.Epilogue) == 40
    assert trt.Epilogue.row_scale.offset == 32


def test_output_dtypes_accepted():
    for i in (trt.F16, trt.BF16):
        for o in (trt.F16, trt.BF16, trt.F32):
            assert status(in_dtype=i, out_dtype=o) == trt.OK, (i, o)
    assert status(in_dtype=trt.F16, out_dtype=4) == trt.ERR_DTYPE


def test_f32_inputs_accepted():
    # binary32 operands with every output dtype
    for o in (trt.F16, trt.BF16, trt.F32):
        assert status(in_dtype=trt.F32, out_dtype=o) == trt.OK, o
    assert status(in_dtype=trt.F32, out_dtype=trt.F32, tile=(128, 128, 32)) == trt.OK


def test_f32_inputs_alignment_extent_and_tile():
    # A and B are aligned to the 4-byte input element
    assert status(in_dtype=trt.F32, A=BASE + 2) == trt.ERR_ALIGN
    assert status(in_dtype=trt.F32, B=BASE * 2 + 2) == trt.ERR_ALIGN
    assert status(in_dtype=trt.F16, A=BASE + 2) == trt.OK
    # A of 4-byte elements spans 4*(63*32 + 32) bytes
    assert status(in_dtype=trt.F32, C=BASE + 4 * 2048) == trt.OK
    assert status(in_dtype=trt.F32, C=BASE + 4 * 2048 - 2) == trt.ERR_OVERLAP
    # transposed B [N][ldb] of 4-byte elements spans 4*(63*ldb + 32)
    assert status(in_dtype=trt.F32, opB=1, ldb=32, C=BASE * 2 + 4 * (63 * 32 + 32)) == trt.OK
    assert status(in_dtype=trt.F32, opB=1, ldb=32,
                  C=BASE * 2 + 4 * (63 * 32 + 32) - 4) == trt.ERR_OVERLAP
    # binary32 operands run on the 128x128x32 tile only
    assert status(in_dtype=trt.F32, tile=(256, 256, 32)) == trt.ERR_UNSUPPORTED
    assert status(in_dtype=trt.F32, tile=(16, 64, 32)) == trt.ERR_UNSUPPORTED


def test_f32_output_alignment_and_extent():
    # C, bias, residual and row scale are aligned to the 4-byte output element
    assert status(out_dtype=trt.F32, C=BASE * 3 + 2) == trt.ERR_ALIGN
    assert status(out_dtype=trt.F32, bias=BASE * 4 + 2) == trt.ERR_ALIGN
    assert status(out_dtype=trt.F32, scale=BASE * 4 + 2) == trt.ERR_ALIGN
    assert status(out_dtype=trt.F16, scale=BASE * 4 + 2) == trt.OK
    # C of 4-byte elements spans 4*(63*64 + 64) bytes
    c_bytes = 4 * (63 * 64 + 64)
    assert status(out_dtype=trt.F32, C=BASE - c_bytes) == trt.OK
    assert status(out_dtype=trt.F32, C=BASE - c_bytes + 4) == trt.ERR_OVERLAP


def test_row_scale_overlap_rejected():
    # the row scale spans M elements of the output type
    assert status(scale=BASE * 3 + 2 * 10) == trt.ERR_OVERLAP
    assert status(scale=BASE * 3 - 2 * 64) == trt.OK          # ends where C starts
    assert status(scale=BASE * 3 - 2 * 64 + 2) == trt.ERR_OVERLAP
    assert status(out_dtype=trt.F32, scale=BASE * 3 - 4 * 64 + 4) == trt.ERR_OVERLAP


# ---- the GF(2) layout algebra of the library against the oracle's ------------------

def _rand_cols(rng, nin, nout, zero_frac=0.0):
    return [0 if rng.random() < zero_frac else (int(rng.integers(0, 1 << nout)) if nout else 0)
            for _ in range(nin)]


def test_gf2_algebra_matches_oracle():
    rng = np.random.default_rng(41)
    for _ in range(200):
        a_in, a_out, b_in, b_out = (int(v) for v in rng.integers(0, 9, 4))
        a = _rand_cols(rng, a_in, a_out, 0.2)
        b = _rand_cols(rng, b_in, b_out, 0.2)
        assert trt.gf2_rank(a, a_out) == L.lin_rank(a, a_out)
        assert trt.gf2_product(a, a_out, b, b_out) == L.lin_product(a, a_out, b)
        outer = _rand_cols(rng, a_out, b_out)
        assert trt.gf2_compose(outer, b_out, a, a_out) == L.lin_compose(outer, a)
        in_mask, out_mask = int(rng.integers(0, 1 << 9)), int(rng.integers(0, 1 << 9))
        cols, ni, no = trt.gf2_sublayout(a, a_out, in_mask, out_mask)
        ins = [i for i in range(a_in) if (in_mask >> i) & 1]
        outs = [o for o in range(a_out) if (out_mask >> o) & 1]
        assert (cols, ni, no) == (L.lin_sublayout(a, a_out, ins, outs), len(ins), len(outs))


def test_gf2_invert_and_compose_matches_oracle():
    rng = np.random.default_rng(42)
    solved = 0
    for _ in range(300):
        nr, ns, nt = int(rng.integers(0, 8)), int(rng.integers(0, 9)), int(rng.integers(0, 8))
        S = _rand_cols(rng, ns, nt, 0.25)
        if ns and rng.random() < 0.3:
            S[int(rng.integers(0, ns))] = S[0]
        R = _rand_cols(rng, nr, nt)
        ref = L.lin_invert_and_compose(R, S, nt)
        if ref is None:
            with pytest.raises(trt.TrtError) as e:
                trt.gf2_invert_and_compose(R, S, nt)
            assert e.value.status == trt.ERR_ARG
        else:
            # the same particular solution: pivots on the first independent columns
            assert trt.gf2_invert_and_compose(R, S, nt) == ref
            solved += 1
    assert solved > 100


def test_gf2_argument_errors():
    with pytest.raises(trt.TrtError) as e:
        trt.gf2_compose([1, 2], 2, [1], 1)          # outer has 2 input bits, inner 1 output bit
    assert e.value.status == trt.ERR_ARG
    with pytest.raises(trt.TrtError):
        trt.gf2_product([1] * 20, 1, [1] * 20, 1)   # 40 input bits
    assert trt.lib().trt_gf2_rank(1, 2, trt._u32([4])) == -1   # column beyond nout
    with pytest.raises(trt.TrtError):
        trt.gf2_rank([0] * 33, 4)


# ---- the block reduction: argument checks (no HIP call on error) -------------------

@pytest.mark.parametrize("kw,code", [
    (dict(n=0), trt.ERR_SIZE), (dict(block=0), trt.ERR_SIZE), (dict(n=(1 << 40) + 1), trt.ERR_SIZE),
    (dict(dtype=4), trt.ERR_DTYPE), (dict(op=3), trt.ERR_ARG),
    (dict(x=0), trt.ERR_NULL), (dict(out=0), trt.ERR_NULL),
    (dict(x=BASE + 1), trt.ERR_ALIGN), (dict(dtype=trt.F32, x=BASE + 2), trt.ERR_ALIGN),
    (dict(out=BASE * 2 + 2), trt.ERR_ALIGN),
    (dict(out=BASE + 1000), trt.ERR_OVERLAP),          # inside x (4096 f16 = 8 KiB)
    (dict(out=BASE - 4 * 64 + 4), trt.ERR_OVERLAP),    # 64 results end inside x
])
def test_block_reduce_rejections(kw, code):
    a = dict(x=BASE, n=4096, block=64, dtype=trt.F16, op=trt.REDUCE_SUM, out=BASE * 2)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.block_reduce_raw(a["x"], a["n"], a["block"], a["dtype"], a["op"], a["out"])
    assert e.value.status == code
    assert trt.last_error() != ""


# ---- register tiles of any logical shape ("My Triton From Scratch, Part 16:
# Register Tiles", sections "Choosing the physical thread shape" and "A strided
# ownership rule") ---------------------------------------------------------------

def test_regtile_policy_matches_pages(golden):
    g = golden("dot_policy.json")
    for out, threads, regs in g["table"]:
        tm, tn = trt.regtile_thread_shape(out[0], out[1], g["max_threads"])
        assert (tm, tn) == tuple(threads), out
        assert (out[0] // tm, out[1] // tn) == tuple(regs), out


@pytest.mark.parametrize("max_threads", [1, 6, 32, 64])
def test_regtile_policy_matches_oracle(max_threads):
    for lm in range(1, 41):
        for ln in list(range(1, 41)) + [64, 96, 100, 127, 128, 192, 512]:
            assert trt.regtile_thread_shape(lm, ln, max_threads) == \
                L.dot_thread_shape((lm, ln), max_threads), (lm, ln)


@pytest.mark.parametrize("lm,ln,mt", [(3, 17, 32), (3, 17, 64), (8, 8, 32), (16, 32, 32),
                                      (48, 80, 64), (64, 64, 64), (5, 7, 64), (1, 64, 32),
                                      (96, 1, 64), (24, 40, 64)])
def test_regtile_owner_matches_oracle(lm, ln, mt):
    tm, tn = trt.regtile_thread_shape(lm, ln, mt)
    rm, rn = lm // tm, ln // tn
    rows, cols = trt.regtile_owner(lm, ln, tm, tn)
    exp = [L.regtile_coordinate((lm, ln), (tm, tn), (t // tn, t % tn), (r // rn, r % rn))
           for t in range(tm * tn) for r in range(rm * rn)]
    assert list(zip(rows.tolist(), cols.tolist())) == exp
    # exactly once
    assert len(set(exp)) == lm * ln


def test_regtile_errors():
    import ctypes
    lib = trt.lib()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    assert lib.trt_regtile_thread_shape(0, 4, 32, ctypes.byref(a), ctypes.byref(b)) == trt.ERR_SIZE
    assert lib.trt_regtile_thread_shape(4, 4, 0, ctypes.byref(a), ctypes.byref(b)) == trt.ERR_ARG
    assert lib.trt_regtile_thread_shape(4, 4, 32, None, ctypes.byref(b)) == trt.ERR_NULL
    buf = np.zeros(64, dtype=np.int32)
    p = buf.ctypes.data
    assert lib.trt_regtile_owner(8, 8, 3, 8, p, p, 64) == trt.ERR_ARG      # 3 does not divide 8
    assert lib.trt_regtile_owner(8, 8, 4, 8, p, p, 63) == trt.ERR_SIZE
    assert lib.trt_regtile_owner(8, 8, 4, 8, None, p, 64) == trt.ERR_NULL
    assert lib.trt_regtile_owner(8, 0, 4, 8, p, p, 0) == trt.ERR_SIZE


@pytest.mark.parametrize("kw,code", [
    (dict(lm=0), trt.ERR_SIZE), (dict(max_threads=0), trt.ERR_ARG),
    (dict(max_threads=65), trt.ERR_ARG),
    (dict(lm=128, ln=128), trt.ERR_UNSUPPORTED),        # (8, 8) threads -> 16 registers per axis
    (dict(lm=9, ln=1, max_threads=1), trt.ERR_UNSUPPORTED),
    (dict(M=0), trt.ERR_SIZE), (dict(in_dtype=5), trt.ERR_DTYPE),
    (dict(C=BASE), trt.ERR_OVERLAP),
])
def test_gemm_regtile_errors_before_device_work(kw, code):
    a = dict(M=64, N=64, K=32, A=BASE, lda=32, opA=0, B=BASE * 2, ldb=64, opB=0,
             C=BASE * 3, ldc=64, in_dtype=trt.F16, out_dtype=trt.F16, lm=16, ln=16,
             max_threads=64)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.gemm_regtile_raw(a["M"], a["N"], a["K"], a["A"], a["lda"], a["opA"], a["B"],
                             a["ldb"], a["opB"], a["C"], a["ldc"], a["in_dtype"],
                             a["out_dtype"], a["lm"], a["ln"], a["max_threads"])
    assert e.value.status == code


def test_torch_wrapper_checks_epilogue_operands():
    # the torch-level wrappers refuse mismatched epilogue operands before any
    # device work (CPU tensors suffice: nothing reaches the library)
    import torch
    A = torch.zeros(8, 4, dtype=torch.float16)
    B = torch.zeros(4, 6, dtype=torch.float16)
    for fn in (trt.gemm, lambda *a, **k: trt.gemm_regtile(*a, lm=4, ln=6, **k)):
        with pytest.raises(trt.TrtError) as e:
            fn(A, B, bias=torch.zeros(6, dtype=torch.float32))
        assert e.value.status == trt.ERR_DTYPE
        with pytest.raises(trt.TrtError) as e:
            fn(A, B, bias=torch.zeros(5, dtype=torch.float16))
        assert e.value.status == trt.ERR_SIZE
        with pytest.raises(trt.TrtError) as e:
            fn(A, B, residual=torch.zeros(8, 5, dtype=torch.float16))
        assert e.value.status == trt.ERR_SIZE
        with pytest.raises(trt.TrtError) as e:
            fn(A, B, row_scale=torch.zeros(8, dtype=torch.bfloat16))
        assert e.value.status == trt.ERR_DTYPE
        with pytest.raises(trt.TrtError) as e:
            fn(A, torch.zeros(5, 6, dtype=torch.float16))
        assert e.value.status == trt.ERR_SIZE


# ---- tile choice (host logic) --------------------------------------------------

def _expected_tile(M, N):
    """The documented rule of trt_choose_tile, restated."""
    cdiv = lambda a, b: -(-a // b)
    if M <= 16:
        return (16, 64, 256)
    count = lambda bm, bn: cdiv(M, bm) * cdiv(N, bn)
    cost = lambda bm, bn: cdiv(count(bm, bn), 256) * bm * bn
    if count(256, 256) >= 192 or count(256, 192) >= 192:
        return (256, 192, 32) if cost(256, 192) < cost(256, 256) else (256, 256, 32)
    if count(128, 128) >= 64:
        return (128, 128, 32)
    return (64, 64, 64)


def test_choose_tile_named_workloads():
    assert trt.choose_tile(4096, 4096) == (256, 256, 32)          # square
    assert trt.choose_tile(8192, 8192, trt.BF16) == (256, 256, 32)  # epilogue
    assert trt.choose_tile(4000, 3072) == (256, 192, 32)          # ragged: one full round
    assert trt.choose_tile(16, 16384) == (16, 64, 256)            # skinny
    assert trt.choose_tile(64, 64) == (64, 64, 64)                # tiny (runs its own tile explicitly)
    assert trt.choose_tile(2048, 2048) == (128, 128, 32)          # mid-size: pipelined 128x128
    assert trt.choose_tile(1024, 1024) == (128, 128, 32)
    assert trt.choose_tile(896, 896) == (64, 64, 64)                # 49 tiles of 128x128
    assert trt.choose_tile(4096, 4096, trt.F32) == (128, 128, 32)


def test_choose_tile_matches_rule():
    rng = np.random.default_rng(11)
    for _ in range(2000):
        M, N = int(rng.integers(1, 20000)), int(rng.integers(1, 20000))
        assert trt.choose_tile(M, N) == _expected_tile(M, N), (M, N)


def test_choose_tile_errors():
    import ctypes
    t = trt.TileDesc()
    assert trt.lib().trt_choose_tile(0, 4, trt.F16, ctypes.byref(t)) == trt.ERR_SIZE
    assert trt.lib().trt_choose_tile(4, 4, 7, ctypes.byref(t)) == trt.ERR_DTYPE
    assert trt.lib().trt_choose_tile(4, 4, trt.F16, None) == trt.ERR_NULL


# ---- the split-K streaming path's workspace (trt_gemm_ws) -------------------------

def test_workspace_size():
    # the skinny workload: 64 panels of 256 columns, 8 slices of 64 iterations
    assert trt.workspace_size(16, 16384, 16384) == 8 * 16 * 16384 * 4
    assert trt.workspace_size(5, 1000, 8192) > 0
    # shapes that never split: M > 16, transposed storage, binary32 inputs, short K,
    # K or N off the vector grid
    assert trt.workspace_size(17, 16384, 16384) == 0
    assert trt.workspace_size(16, 16384, 16384, opA=trt.OP_T) == 0
    assert trt.workspace_size(16, 16384, 16384, opB=trt.OP_T) == 0
    assert trt.workspace_size(16, 16384, 16384, in_dtype=trt.F32) == 0
    assert trt.workspace_size(16, 16384, 256) == 0
    assert trt.workspace_size(16, 16384, 16380) == 0
    assert trt.workspace_size(16, 16382, 16384) == 0
    for bad in [dict(M=0), dict(K=1 << 31), dict(opA=2), dict(in_dtype=9)]:
        a = dict(M=16, N=64, K=4096, opA=0, opB=0, in_dtype=trt.F16)
        a.update(bad)
        with pytest.raises(trt.TrtError):
            trt.workspace_size(a["M"], a["N"], a["K"], a["opA"], a["opB"], a["in_dtype"])


GIB = 1 << 30     # fake addresses far apart: B alone spans 512 MiB here


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=0), trt.ERR_NULL),
    (dict(workspace_bytes=8 * 16 * 16384 * 4 - 16), trt.ERR_SIZE),
    (dict(workspace=8 * GIB + 8), trt.ERR_ALIGN),
    (dict(workspace=4 * GIB + 4096), trt.ERR_OVERLAP),      # inside C
    (dict(workspace=2 * GIB - 4096), trt.ERR_OVERLAP),      # reaches into B from below
    (dict(workspace=2 * GIB + 4096), trt.ERR_OVERLAP),      # inside B
    (dict(workspace=GIB - 4096), trt.ERR_OVERLAP),          # reaches into A
])
def test_gemm_ws_workspace_errors(kw, code):
    # every case returns before any HIP call (no GPU is needed)
    M, N, K = 16, 16384, 16384
    a = dict(workspace=8 * GIB, workspace_bytes=8 * 16 * 16384 * 4)
    a.update(kw)
    with pytest.raises(trt.TrtError) as e:
        trt.gemm_ws_raw(M, N, K, GIB, K, 0, 2 * GIB, N, 0, 4 * GIB, N, trt.F16, trt.F16,
                        workspace=a["workspace"], workspace_bytes=a["workspace_bytes"])
    assert e.value.status == code, trt.last_error()
    assert "workspace" in trt.last_error()
