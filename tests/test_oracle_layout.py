"""Pins of the layout oracle: the values the pages print, and invariants.

Every fixture under tests/golden/ names the page and section it comes from.
"""
import itertools

import numpy as np
import pytest

from oracle import layout_ref as L


# ---- Part 12: cooperative traversal ---------------------------------------

@pytest.mark.parametrize("name", ["coop_a_4x16.json", "coop_b_16x8.json"])
def test_cooperative_examples(golden, name):
    g = golden(name)
    shape, T, order = tuple(g["logical_shape"]), g["threads"], tuple(g["order"])
    assert L.coop_iterations(shape, T) == g["iterations"]
    for t, i, lin, coord in g["visits"]:
        assert L.coop_linear(shape, T, t, i) == lin
        assert L.coop_coordinate(shape, order, lin) == tuple(coord)
    # every element covered exactly once
    seen = [L.coop_coordinate(shape, order, L.coop_linear(shape, T, t, i))
            for t in range(T) for i in range(g["iterations"])
            if L.coop_contains(shape, T, t, i)]
    assert len(seen) == len(set(seen)) == g["size"]


def test_cooperative_tail_lanes_inactive():
    # a tile smaller than the block: only the first `size` threads are active
    shape, T = (3, 5), 32
    assert L.coop_iterations(shape, T) == 1
    active = [t for t in range(T) if L.coop_contains(shape, T, t, 0)]
    assert active == list(range(15))


def test_cooperative_order_column_major():
    # order (0, 1): axis 0 changes fastest
    assert L.coop_coordinate((4, 16), (0, 1), 1) == (1, 0)
    assert L.coop_coordinate((4, 16), (0, 1), 4) == (0, 1)


@pytest.mark.parametrize("bad", [
    lambda: L.coop_iterations((4, 16), 0),
    lambda: L.coop_iterations((4, 16), 1025),
    lambda: L.coop_linear((4, 16), 32, 32, 0),
    lambda: L.coop_linear((4, 16), 32, 0, 2),
    lambda: L.coop_coordinate((4, 16), (1, 1), 0),
    lambda: L.coop_coordinate((4, 16), (1, 0), 64),
    lambda: L.coop_coordinate((4, 0), (1, 0), 0),
    lambda: L.coop_coordinate((1, 2, 3), (0, 1, 2), 0),
])
def test_cooperative_validation(bad):
    with pytest.raises(ValueError):
        bad()


# ---- Part 12: kernel layouts and projections --------------------------------

def test_kernel_layouts(golden):
    g = golden("kernel_layouts.json")
    for c in g["kernel_layouts"]:
        kl = L.kernel_layout(tuple(c["output"]), tuple(c["thread"]))
        assert kl == {"rank": c["rank"], "is_rank2": c["is_rank2"],
                      "threads_per_block": c["threads_per_block"]}
    for c in g["projections"]:
        got = L.tile_layout(tuple(c["thread"]), tuple(c["logical"]),
                            tuple(c["broadcast_axes"]))
        assert got == tuple(c["thread_axes"])
    for c in g["rejected_projections"]:
        with pytest.raises(ValueError):
            L.tile_layout(tuple(c["thread"]), tuple(c["logical"]))


@pytest.mark.parametrize("out,thr", [((4, 8), (4,)), ((64, 64), (32, 64)),
                                     ((0, 8), (4, 8)), ((4, 8), (4, -8))])
def test_kernel_layout_rejects(out, thr):
    with pytest.raises(ValueError):
        L.kernel_layout(out, thr)


# ---- Part 16: register tiles ---------------------------------------------------

def test_regtile_examples(golden):
    for c in golden("regtile_examples.json")["cases"]:
        lg, th = tuple(c["logical"]), tuple(c["thread"])
        assert L.register_shape(lg, th) == tuple(c["register_shape"])
        assert L.registers_per_thread(lg, th) == c["registers_per_thread"]
        for reg, logical in c["owns"]:
            assert L.regtile_coordinate(lg, th, tuple(c["thread_coord"]),
                                        tuple(reg)) == tuple(logical)


@pytest.mark.parametrize("lg,th", [((8, 8), (4, 8)), ((16, 16), (4, 8)),
                                   ((16, 32), (4, 8)), ((3, 17), (1, 17))])
def test_regtile_exactly_once(lg, th):
    rs = L.register_shape(lg, th)
    owned = [L.regtile_coordinate(lg, th, (ti, tj), (ri, rj))
             for ti in range(th[0]) for tj in range(th[1])
             for ri in range(rs[0]) for rj in range(rs[1])]
    assert len(owned) == len(set(owned)) == lg[0] * lg[1]


def test_regtile_rejects():
    with pytest.raises(ValueError):
        L.register_shape((8, 8), (3, 8))
    with pytest.raises(ValueError):
        L.register_shape((8,), (4,))
    with pytest.raises(ValueError):
        L.regtile_coordinate((8, 8), (4, 8), (4, 0), (0, 0))
    with pytest.raises(ValueError):
        L.regtile_coordinate((8, 8), (4, 8), (0, 0), (2, 0))


def test_dot_policy_table(golden):
    g = golden("dot_policy.json")
    for out, threads, regs in g["table"]:
        th = L.dot_thread_shape(tuple(out), g["max_threads"])
        assert th == tuple(threads)
        assert L.register_shape(tuple(out), th) == tuple(regs)


# ---- Triton LinearLayout: GF(2) maps ----------------------------------------

def test_gf2_lane_warp_example(golden):
    g = golden("gf2_examples.json")["lane_warp"]
    bases = {k: [tuple(v) for v in vs] for k, vs in g["bases"].items()}
    for ins, out in g["apply"]:
        assert L.gf2_apply(bases, ins) == tuple(out)
    # closed form over the whole 4x4 input space
    for lane, warp in itertools.product(range(4), range(4)):
        assert L.gf2_apply(bases, {"lane": lane, "warp": warp}) == (lane, lane ^ warp)
    assert L.gf2_is_injective(bases, g["out_bits"])
    assert L.gf2_is_surjective(bases, g["out_bits"])


def test_gf2_blocked_example(golden):
    g = golden("gf2_examples.json")["blocked"]
    bases = {k: [tuple(v) for v in vs] for k, vs in g["bases"].items()}
    for ins, out in g["apply"]:
        assert L.gf2_apply(bases, ins) == tuple(out)
    outs = {L.gf2_apply(bases, {"register": r, "lane": l, "warp": w})
            for r in range(8) for l in range(32) for w in range(4)}
    assert len(outs) == g["coverage"]
    assert L.gf2_rank(bases, g["out_bits"]) == 10


def test_gf2_rank_detects_broadcast():
    # a zero basis is a broadcast: not injective; duplicated basis: rank drops
    bases = {"lane": [(1, 0), (2, 0)], "warp": [(0, 0)]}
    assert not L.gf2_is_injective(bases, [2, 1])
    assert not L.gf2_is_surjective(bases, [2, 1])
    dup = {"lane": [(1, 1), (1, 1)]}
    assert L.gf2_rank(dup, [1, 1]) == 1


def test_gf2_rank_brute_force():
    # rank == log2(|image|) on random small layouts
    import random
    rnd = random.Random(7)
    for _ in range(200):
        n_in = rnd.randint(1, 6)
        vecs = [(rnd.randrange(8), rnd.randrange(4)) for _ in range(n_in)]
        bases = {"x": vecs}
        image = {L.gf2_apply(bases, {"x": v}) for v in range(1 << n_in)}
        assert 1 << L.gf2_rank(bases, [3, 2]) == len(image)


# ---- MI355X maps ---------------------------------------------------------------

def test_mfma16_maps_are_bijections():
    a = {L.mfma16_a(l, e) for l in range(64) for e in range(8)}
    b = {L.mfma16_b(l, e) for l in range(64) for e in range(8)}
    c = {L.mfma16_c(l, r) for l in range(64) for r in range(4)}
    assert a == {(i, k) for i in range(16) for k in range(32)}
    assert b == {(k, j) for k in range(32) for j in range(16)}
    assert c == {(i, j) for i in range(16) for j in range(16)}
    # A and B pair the same k in the same (lane group, element) slot
    for l in range(64):
        for e in range(8):
            assert L.mfma16_a(l, e)[1] == L.mfma16_b(l, e)[0]


def test_mfma16f32_maps_are_bijections():
    a = {L.mfma16f32_a(l) for l in range(64)}
    b = {L.mfma16f32_b(l) for l in range(64)}
    assert a == {(i, k) for i in range(16) for k in range(4)}
    assert b == {(k, j) for k in range(4) for j in range(16)}
    for l in range(64):
        assert L.mfma16f32_a(l)[1] == L.mfma16f32_b(l)[0]


# The library's compiled power-of-two tiles (BM, BN, BK, waves along m, waves
# along n), all on 16x16 fragments, and one tile of 32x32 fragments: the
# probe's second fragment shape, whose result map the one-hot test pins.
TILE_CONFIGS = [(16, 64, 32, 1, 1), (64, 64, 64, 2, 2), (128, 128, 64, 2, 2),
                (256, 256, 64, 2, 2), (256, 256, 32, 2, 4), (256, 256, 32, 2, 2),
                (128, 128, 32, 2, 2), (128, 128, 32, 2, 2, 32)]


@pytest.mark.parametrize("cfg", TILE_CONFIGS)
def test_gemm_c_owner_exactly_once(cfg):
    BM, BN, BK, WM, WN = cfg[:5]
    regs = L.gemm_regs_per_lane(cfg)
    owned = [L.gemm_c_owner(cfg, r, l, w)
             for w in range(WM * WN) for l in range(64) for r in range(regs)]
    assert len(owned) == len(set(owned)) == BM * BN
    assert all(0 <= i < BM and 0 <= j < BN for i, j in owned)


@pytest.mark.parametrize("cfg", TILE_CONFIGS)
def test_gemm_c_owner_is_gf2_linear(cfg):
    BM, BN, BK, WM, WN = cfg[:5]
    bases = L.gemm_c_bases(cfg)
    out_bits = [L.log2_exact(BM), L.log2_exact(BN)]
    assert L.gf2_is_injective(bases, out_bits) and L.gf2_is_surjective(bases, out_bits)
    regs = L.gemm_regs_per_lane(cfg)
    for w in range(WM * WN):
        for l in range(64):
            for r in range(regs):
                assert L.gemm_c_owner(cfg, r, l, w) == L.gf2_apply(
                    bases, {"reg": r, "lane": l, "wave": w})


def test_tiny_tile_owner_values():
    # the 16x64 tile over one wave: lane 17 (row 1, column group 1), reg 6
    # (fragment 1, register 2) -> C(1, 16 + 4 + 2)
    assert L.gemm_c_owner((16, 64, 32, 1, 1), 6, 17, 0) == (1, 22)
    assert L.gemm_regs_per_lane((16, 64, 32, 1, 1)) == 16


@pytest.mark.parametrize("R,G", [(16, 4), (64, 4), (64, 8), (256, 8), (128, 8)])
def test_lds_slot_bijective(R, G):
    slots = {L.lds_slot(r, g, G) for r in range(R) for g in range(G)}
    assert slots == set(range(R * G))


def _conflicts(addresses, banks=32):
    """Worst number of distinct 16-byte chunks sharing a bank group among
    lanes that a 16-byte-per-lane LDS access serves in one cycle."""
    worst = 1
    lanes_per_cycle = banks * 4 // 16
    for base in range(0, len(addresses), lanes_per_cycle):
        grp = addresses[base:base + lanes_per_cycle]
        col = {}
        for a in grp:
            col.setdefault((a // 16) % lanes_per_cycle, set()).add(a)
        worst = max(worst, max(len(v) for v in col.values()))
    return worst


@pytest.mark.parametrize("R,G", [(64, 4), (256, 8), (128, 8)])
def test_lds_swizzle_conflict_free_reads(R, G):
    # fragment read: 16 consecutive rows, one k chunk, per 16 lanes
    for r0 in range(0, R, 16):
        for g in range(G):
            addrs = [16 * L.lds_slot(r0 + (l % 16), g, G) for l in range(16)]
            assert _conflicts(addrs, 32) == 1


# Epilogue staging of the pipelined tiles (BM, BN, WM, WN): one pass holds
# BM/2 rows; the tile row of a fragment element goes to staged row
# (row // WTM) * (WTM/2) + row % (WTM/2).  Byte address of the 16-byte column
# group c/4 of staged row r: swizzled (group XOR r mod 16, rows of BN floats),
# or padded (rows of BN + pad floats, no XOR) as the kernel used to stage.
STAGING_TILES = [(256, 256, 2, 4), (256, 192, 2, 2), (128, 128, 2, 2)]


def _stage_addr(BN, r, c, pad=None):
    if pad is None:
        return 4 * (r * BN + 4 * ((c // 4) ^ (r % 16)))
    return 4 * (r * (BN + pad) + c)


def _staging_store_addrs(tile, wave, fm, fn, pad=None):
    BM, BN, WM, WN = tile
    WTM = BM // WM
    cfg = (BM, BN, 32, WM, WN, 16)
    FN = (BN // WN) // 16
    out = []
    for lane in range(64):
        row, col = L.gemm_c_owner(cfg, 4 * (fm * FN + fn), lane, wave)
        out.append(_stage_addr(BN, (row // WTM) * (WTM // 2) + row % (WTM // 2), col, pad))
    return out


def _staging_read_addrs(tile, it, wave, pad=None):
    # the store phase: PANEL columns per item (the row when BN is a power of
    # two, else 64), PANEL/4 threads per row, four columns per thread
    BM, BN, WM, WN = tile
    panel = BN if BN & (BN - 1) == 0 else 64
    panels, tpr = BN // panel, panel // 4
    rows_per_step = 64 * WM * WN // tpr
    out = []
    for lane in range(64):
        t = 64 * wave + lane
        r = (it // panels) * rows_per_step + t // tpr
        c = (it % panels) * panel + 4 * (t % tpr)
        out.append(_stage_addr(BN, r, c, pad))
    return out


@pytest.mark.parametrize("tile", STAGING_TILES)
def test_epilogue_staging_conflict_free(tile):
    # every fragment store and every store-phase read of the swizzled staging
    # serves its 8-lane groups from distinct bank groups
    BM, BN, WM, WN = tile
    FM, FN = (BM // WM) // 16, (BN // WN) // 16
    for wave in range(WM * WN):
        for fm in range(FM):
            for fn in range(FN):
                assert _conflicts(_staging_store_addrs(tile, wave, fm, fn), 32) == 1
        for it in range(4 * (BN // 64)):
            assert _conflicts(_staging_read_addrs(tile, it, wave), 32) == 1


def test_epilogue_staging_model_matches_padded_counts():
    # The same model on the padded layout the kernel used before: stores of
    # rows padded by 4 floats are conflict-free, by 8 floats 2-way and by 16
    # floats 4-way in every 8-lane group -- on the 256x256 tile the counter
    # read 0, 8 and 24 extra cycles per fragment store for paddings of 4 (or
    # 12), 8 and 16 floats.  (The padded 256x192 layout's store-phase reads
    # also cost 4 extra cycles each on the hardware; this model does not see
    # those, the swizzled layout measures 0 on every tile.)
    tile = (256, 256, 2, 4)
    for pad, ways in ((4, 1), (12, 1), (8, 2), (16, 4)):
        assert _conflicts(_staging_store_addrs(tile, 0, 0, 0, pad), 32) == ways


# binary32 operand tiles: rows of 32 floats (eight 16-byte chunks), chunk kc
# of row r at position kc ^ sw(r); a fragment read gives lane l row
# (l % 16) of a 16-row block and chunk 2 (l // 16) + h.
def _f32_read_addrs(sw, r0, h):
    return [128 * (r0 + l % 16) + 16 * ((2 * (l // 16) + h) ^ sw(r0 + l % 16)) for l in range(64)]


def test_f32_staging_conflict_free():
    sw = lambda r: (r ^ (r >> 3)) & 7
    for r0 in range(0, 128, 16):
        for h in range(2):
            assert _conflicts(_f32_read_addrs(sw, r0, h), 32) == 1
    # the copies of rows-contiguous storage: eight lanes write rows 4 apart
    for i in range(4):
        for t0 in range(0, 256, 8):
            addrs = [128 * (4 * (t % 32) + i) + 16 * ((t // 32) ^ sw(4 * (t % 32) + i))
                     for t in range(t0, t0 + 8)]
            assert _conflicts(addrs, 32) == 1
    # the swizzle on row bits 1-3 that the counter measured at 16.8 M conflict
    # cycles per 4096^3 launch: row pairs share a position, 2-way
    old = lambda r: ((r >> 1) ^ (r >> 3)) & 7
    assert _conflicts(_f32_read_addrs(old, 0, 0), 32) == 2


@pytest.mark.parametrize("R,G,T", [(256, 8, 256), (64, 4, 64), (128, 8, 256)])
def test_lds_swizzle_conflict_free_writes(R, G, T):
    # k-contiguous copy: each thread writes its chunk (r, g)
    for i in range(-(-R * G // T)):
        addrs = []
        for t in range(T):
            c = L.copy_kcontig(R, G, T, t, i)
            if c is not None:
                addrs.append(16 * L.lds_slot(c[0], c[1], G))
        assert _conflicts(addrs, 32) == 1
    # row-contiguous copy: block (rb, g), write j lands on row 8rb + j.  With
    # four chunks per row (64-byte rows) a bank window holds two rows, and the
    # eight lanes of a cycle all write rows of one parity: two-way at best.
    worst = 1 if G == 8 else 2
    for i in range(-(-(R // 8) * G // T)):
        for j in range(8):
            addrs = []
            for t in range(T):
                c = L.copy_mncontig(R, G, T, t, i)
                if c is not None:
                    addrs.append(16 * L.lds_slot(8 * c[0] + j, c[1], G))
            assert _conflicts(addrs, 32) <= worst


def test_copy_maps_cover_tile():
    for R, G, T in [(256, 8, 256), (16, 4, 64), (64, 4, 64)]:
        it = -(-R * G // T)
        got = [L.copy_kcontig(R, G, T, t, i) for t in range(T) for i in range(it)]
        got = [x for x in got if x is not None]
        assert sorted(got) == [(r, g) for r in range(R) for g in range(G)]
        it = -(-(R // 8) * G // T)
        got = [L.copy_mncontig(R, G, T, t, i) for t in range(T) for i in range(it)]
        got = [x for x in got if x is not None]
        assert sorted(got) == [(rb, g) for rb in range(R // 8) for g in range(G)]


def test_mfma32_maps_are_bijections():
    a = {L.mfma32_a(l, e) for l in range(64) for e in range(8)}
    b = {L.mfma32_b(l, e) for l in range(64) for e in range(8)}
    c = {L.mfma32_c(l, r) for l in range(64) for r in range(16)}
    assert a == {(i, k) for i in range(32) for k in range(16)}
    assert b == {(k, j) for k in range(16) for j in range(32)}
    assert c == {(i, j) for i in range(32) for j in range(32)}
    for l in range(64):
        for e in range(8):
            assert L.mfma32_a(l, e)[1] == L.mfma32_b(l, e)[0]


def test_owner_runs_of_four_columns():
    # every run of four consecutive registers holds four consecutive columns
    # of one row: the epilogue's 8-byte vector stores rely on it
    for cfg in [(16, 64, 32, 1, 1), (256, 256, 32, 2, 2, 16), (256, 256, 32, 2, 4, 16),
                (256, 256, 32, 2, 2, 32)]:
        for w in range(cfg[3] * cfg[4]):
            for l in range(64):
                for r0 in range(0, L.gemm_regs_per_lane(cfg), 4):
                    pts = [L.gemm_c_owner(cfg, r0 + e, l, w) for e in range(4)]
                    assert all(p[0] == pts[0][0] for p in pts)
                    assert [p[1] - pts[0][1] for p in pts] == [0, 1, 2, 3]


# ---- direct-to-LDS tiles ---------------------------------------------------------

@pytest.mark.parametrize("cfg", [(256, 192, 32, 2, 4, 16), (256, 192, 32, 2, 2, 16),
                                 (256, 192, 32, 2, 2, 32)])
def test_non_power_of_two_tile_owned_exactly_once(cfg):
    # the 256x192 pipelined tile: 2x4 waves of 128x48, 8x3 fragments of 16x16
    # (or 2x2 waves of 128x96); its ownership is integer-affine, not
    # GF(2)-linear, so it is checked by enumeration ("My Triton From Scratch,
    # Part 16: Register Tiles", section "A strided ownership rule")
    regs = L.gemm_regs_per_lane(cfg)
    assert regs * cfg[3] * cfg[4] * 64 == 256 * 192
    seen = set()
    for w in range(cfg[3] * cfg[4]):
        for l in range(64):
            for r in range(regs):
                seen.add(L.gemm_c_owner(cfg, r, l, w))
    assert len(seen) == 256 * 192 and seen == {(i, j) for i in range(256) for j in range(192)}

@pytest.mark.parametrize("R", [128, 192, 256])
def test_dma_slots_bijective(R):
    assert sorted(L.dma_kc_slot(r, g) for r in range(R) for g in range(4)) == list(range(4 * R))
    assert sorted(L.dma_mn_slot(R, k, c) for k in range(32) for c in range(R // 8)) \
        == list(range(4 * R))


def _conflicts_bytes(addr_bytes, window):
    """Worst count of accesses hitting the same bank among a group of
    accesses served together; banks are 4 bytes wide, window bytes per cycle.
    addr_bytes: list of (start, length) per lane."""
    banks = {}
    for a, n in addr_bytes:
        for b in range(a, a + n, 4):
            banks.setdefault((b % window) // 4, set()).add(b)
    return max(len(v) for v in banks.values())


KCHUNK = (0, 3, 1, 2)     # k chunk of lane group l//16 in the 16x16x32 fragment reads


def test_fragment_chunk_order():
    # a permutation, and the two lane groups reading the same rows (g, g+1)
    # take chunks differing in both bits -- on gfx950 the only pairing whose
    # 16-byte reads cost no extra LDS cycles whatever the swizzle
    assert sorted(KCHUNK) == [0, 1, 2, 3]
    assert KCHUNK[0] ^ KCHUNK[1] == 3 and KCHUNK[2] ^ KCHUNK[3] == 3


@pytest.mark.parametrize("R", [192, 256])
def test_dma_kc_fragment_reads_conflict_free(R):
    # 16x16x32 operand read: lane l reads row rbase + l%16, chunk KCHUNK[l//16]
    for rbase in range(0, R, 16):
        lanes = [(16 * L.dma_kc_slot(rbase + l % 16, KCHUNK[l // 16]), 16) for l in range(64)]
        for n, window in [(8, 128), (16, 256)]:
            for q in range(0, 64, n):
                assert _conflicts_bytes(lanes[q:q + n], window) == 1


@pytest.mark.parametrize("R", [192, 256])
def test_dma_mn_transposed_reads_conflict_free(R):
    # transposing read of a 16x16x32 operand: lane l (group g = l//16, j =
    # l%16) reads 8 bytes at k row 8*KCHUNK[g] + 4h + j//4, columns c0 + 4*(j%4)
    for c0 in range(0, R, 16):
        for h in range(2):
            lanes = []
            for l in range(64):
                g, j = l // 16, l % 16
                k = 8 * KCHUNK[g] + 4 * h + j // 4
                col = c0 + 4 * (j % 4)
                slot = L.dma_mn_slot(R, k, col // 8)
                lanes.append((16 * slot + 2 * (col % 8), 8))
            for n, window in [(16, 128), (32, 256)]:
                for q in range(0, 64, n):
                    assert _conflicts_bytes(lanes[q:q + n], window) == 1


# ---- the layout algebra ("Triton LinearLayout", sections "Combining layouts" and
# "invertAndCompose: derive data movement"), pinned by enumeration ------------------

def _rand_lin(rng, nin, nout, zero_frac=0.0):
    cols = [int(rng.integers(0, 1 << nout)) if nout else 0 for _ in range(nin)]
    return [0 if rng.random() < zero_frac else c for c in cols]


def test_lin_apply_page_example():
    # lane bits 0-1 -> (1,1), (2,2); warp bits 2-3 -> (0,1), (0,2); outputs
    # packed as row (bits 0-1) | col (bits 2-3).  The page evaluates
    # lane=3, warp=2 to (row=3, col=1).
    cols = [1 | 1 << 2, 2 | 2 << 2, 0 | 1 << 2, 0 | 2 << 2]
    assert L.lin_apply(cols, 3 | 2 << 2) == 3 | 1 << 2
    # and the whole map is (lane, lane XOR warp)
    for lane in range(4):
        for warp in range(4):
            assert L.lin_apply(cols, lane | warp << 2) == lane | (lane ^ warp) << 2


def test_lin_compose_is_function_composition():
    rng = np.random.default_rng(31)
    for _ in range(40):
        nin, nmid, nout = (int(v) for v in rng.integers(0, 7, 3))
        inner = _rand_lin(rng, nin, nmid)
        outer = _rand_lin(rng, nmid, nout)
        comp = L.lin_compose(outer, inner)
        for x in range(1 << nin):
            assert L.lin_apply(comp, x) == L.lin_apply(outer, L.lin_apply(inner, x))


def test_lin_product_is_a_direct_sum():
    rng = np.random.default_rng(32)
    for _ in range(30):
        an, ao, bn, bo = (int(v) for v in rng.integers(0, 5, 4))
        a, b = _rand_lin(rng, an, ao), _rand_lin(rng, bn, bo)
        p = L.lin_product(a, ao, b)
        for xa in range(1 << an):
            for xb in range(1 << bn):
                assert L.lin_apply(p, xa | xb << an) == L.lin_apply(a, xa) | L.lin_apply(b, xb) << ao


def test_lin_sublayout_restricts_and_projects():
    rng = np.random.default_rng(33)
    for _ in range(30):
        nin, nout = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        cols = _rand_lin(rng, nin, nout)
        ins = sorted(int(i) for i in rng.choice(nin, int(rng.integers(0, nin + 1)), replace=False))
        outs = sorted(int(o) for o in rng.choice(nout, int(rng.integers(0, nout + 1)), replace=False))
        sub = L.lin_sublayout(cols, nout, ins, outs)
        for x in range(1 << len(ins)):
            full_x = sum(((x >> k) & 1) << i for k, i in enumerate(ins))
            y = L.lin_apply(cols, full_x)
            assert L.lin_apply(sub, x) == sum(((y >> b) & 1) << k for k, b in enumerate(outs))


def test_lin_rank_counts_distinct_images():
    rng = np.random.default_rng(34)
    for _ in range(40):
        nin, nout = int(rng.integers(0, 7)), int(rng.integers(0, 7))
        cols = _rand_lin(rng, nin, nout, zero_frac=0.2)
        images = {L.lin_apply(cols, x) for x in range(1 << nin)}
        assert 1 << L.lin_rank(cols, nout) == len(images)


def test_lin_invert_and_compose_solves_s_q_equals_r():
    rng = np.random.default_rng(35)
    solved = unsolvable = 0
    for _ in range(80):
        nr, ns, nt = int(rng.integers(0, 6)), int(rng.integers(0, 7)), int(rng.integers(0, 6))
        S = _rand_lin(rng, ns, nt, zero_frac=0.25)          # may broadcast (zero bases)
        if rng.random() < 0.3 and ns:
            S[int(rng.integers(0, ns))] = S[0]              # duplicate: not injective
        R = _rand_lin(rng, nr, nt)
        Q = L.lin_invert_and_compose(R, S, nt)
        span = {L.lin_apply(S, y) for y in range(1 << ns)}
        if Q is None:
            assert any(c not in span for c in R)
            unsolvable += 1
            continue
        solved += 1
        for x in range(1 << nr):
            assert L.lin_apply(S, L.lin_apply(Q, x)) == L.lin_apply(R, x)
    assert solved > 20 and unsolvable > 5


def test_lin_invert_and_compose_page_example():
    # R = S = the page's (lane, warp) -> (lane, lane XOR warp): S^-1 o R = identity
    cols = [1 | 1 << 2, 2 | 2 << 2, 0 | 1 << 2, 0 | 2 << 2]
    assert L.lin_invert_and_compose(cols, cols, 4) == [1, 2, 4, 8]
    # with warp bit 1 broadcast in S (a zero basis), S reaches only half of the
    # 4 x 4 coordinates: (row 0, col 2) is outside its image, (3, 3) inside
    S = [1 | 1 << 2, 2 | 2 << 2, 0 | 1 << 2, 0]
    assert L.lin_invert_and_compose([0 | 2 << 2], S, 4) is None
    Q = L.lin_invert_and_compose([3 | 3 << 2], S, 4)
    assert Q is not None and L.lin_apply(S, Q[0]) == 3 | 3 << 2
