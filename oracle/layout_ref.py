"""Layout oracle: ownership, copy and swizzle maps in plain Python integers.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Every function restates a
formula from the pages, or from the stated design of the MI355X kernel, with
no shared code with the HIP layout module it is compared against.

Page maps
  * cooperative tile layout -- "My Triton From Scratch, Part 12: CUDA Tile
    Layouts", sections "Cooperative tile layouts" and "Validation is part of
    the model";
  * kernel layout and projections -- same page, sections "Kernel layout",
    "Projecting logical values onto threads", "Explicit broadcast axes";
  * register tiles -- "My Triton From Scratch, Part 16: Register Tiles",
    sections "Describing the mapping", "A strided ownership rule" and
    "Choosing the physical thread shape";
  * GF(2) linear layouts -- "Triton LinearLayout", sections "Basis-vector
    representation", "LinearLayout::apply" and "Surjectivity, injectivity,
    and broadcasts";
  * the layout algebra -- same page, sections "Combining layouts" and
    "invertAndCompose: derive data movement" (lin_* functions).

MI355X maps (not on the pages; the matrix-core operand layout is AMD's
documented v_mfma_f32_16x16x32_{f16,bf16} register layout)
  * mfma16_a / mfma16_b / mfma16_c -- one 16x16x32 fragment;
  * gemm_c_owner -- (register, lane, wave) -> (row, col) of a workgroup tile;
  * lds_slot -- the XOR-swizzled 16-byte chunk slot of an operand tile;
  * copy_kcontig / copy_mncontig -- the cooperative global->LDS copy maps.
"""
from math import prod

MAX_THREADS_PER_BLOCK = 1024


# --------------------------------------------------------------------------
# Part 12: kernel layout, projection, cooperative traversal
# --------------------------------------------------------------------------

def _check_shape(shape, what):
    if not isinstance(shape, tuple) or len(shape) not in (1, 2):
        raise ValueError(f"{what} must be a rank-1 or rank-2 tuple")
    for d in shape:
        if not isinstance(d, int) or isinstance(d, bool) or d <= 0:
            raise ValueError(f"{what} dims must be positive integers")


def kernel_layout(output_tile_shape, thread_shape):
    """Program-instance layout: both shapes rank 1 or 2, positive, same rank,
    thread product within the 1024-thread block limit (Part 12, "Kernel
    layout").  Returns rank, is_rank2 and threads_per_block."""
    _check_shape(output_tile_shape, "output_tile_shape")
    _check_shape(thread_shape, "thread_shape")
    if len(output_tile_shape) != len(thread_shape):
        raise ValueError("output and thread shapes must have equal rank")
    tpb = prod(thread_shape)
    if tpb > MAX_THREADS_PER_BLOCK:
        raise ValueError("thread product exceeds the block limit")
    return {"rank": len(thread_shape), "is_rank2": len(thread_shape) == 2,
            "threads_per_block": tpb}


def tile_layout(thread_shape, logical_shape, broadcast_axes=()):
    """Projection of a per-thread logical value onto thread axes (Part 12,
    "Projecting logical values onto threads" and "Explicit broadcast axes"):
    an axis listed as broadcast maps to None; otherwise an extent equal to
    the thread extent maps to that axis, an extent of one maps to None, and
    any other extent is rejected."""
    _check_shape(logical_shape, "logical_shape")
    if len(logical_shape) != len(thread_shape):
        raise ValueError("logical and thread shapes must have equal rank")
    for a in broadcast_axes:
        if not (0 <= a < len(logical_shape)):
            raise ValueError("broadcast axis out of range")
    axes = []
    for axis, (ld, td) in enumerate(zip(logical_shape, thread_shape)):
        if axis in broadcast_axes:
            axes.append(None)
        elif ld == td:
            axes.append(axis)
        elif ld == 1:
            axes.append(None)
        else:
            raise ValueError("logical dim cannot be projected onto threads")
    return tuple(axes)


def coop_iterations(logical_shape, threads):
    """ceil(tile size / threads per block) (Part 12, "Cooperative tile layouts")."""
    _check_shape(logical_shape, "logical_shape")
    if not (1 <= threads <= MAX_THREADS_PER_BLOCK):
        raise ValueError("threads out of range")
    return -(-prod(logical_shape) // threads)


def coop_linear(logical_shape, threads, t, i):
    """Linear index that thread t visits at iteration i: t + i*threads."""
    if not (0 <= t < threads):
        raise ValueError("thread index out of range")
    if not (0 <= i < coop_iterations(logical_shape, threads)):
        raise ValueError("iteration out of range")
    return t + i * threads


def coop_contains(logical_shape, threads, t, i):
    """False for the inactive tail lanes of the last iteration."""
    return coop_linear(logical_shape, threads, t, i) < prod(logical_shape)


def coop_coordinate(logical_shape, order, linear):
    """Coordinate of a linear index: peel axes in `order`, fastest first."""
    _check_shape(logical_shape, "logical_shape")
    if sorted(order) != list(range(len(logical_shape))):
        raise ValueError("order must be a permutation of the axes")
    if not (0 <= linear < prod(logical_shape)):
        raise ValueError("linear index outside the tile")
    coord = [0] * len(logical_shape)
    rem = linear
    for axis in order:
        coord[axis] = rem % logical_shape[axis]
        rem //= logical_shape[axis]
    return tuple(coord)


# --------------------------------------------------------------------------
# Part 16: register tiles and the one-warp thread-shape policy
# --------------------------------------------------------------------------

def register_shape(logical_shape, thread_shape):
    """Elementwise quotient, requiring positive rank-2 shapes that divide."""
    for s in (logical_shape, thread_shape):
        if not isinstance(s, tuple) or len(s) != 2 or any(
                not isinstance(d, int) or d <= 0 for d in s):
            raise ValueError("register tiles need positive rank-2 shapes")
    if any(l % t for l, t in zip(logical_shape, thread_shape)):
        raise ValueError("logical dims must be divisible by thread dims")
    return tuple(l // t for l, t in zip(logical_shape, thread_shape))


def registers_per_thread(logical_shape, thread_shape):
    return prod(register_shape(logical_shape, thread_shape))


def regtile_coordinate(logical_shape, thread_shape, thread_coord, reg_coord):
    """Strided ownership: logical = thread + register * thread_shape, per axis."""
    rs = register_shape(logical_shape, thread_shape)
    for c, lim in zip(thread_coord, thread_shape):
        if not (0 <= c < lim):
            raise ValueError("thread coordinate out of range")
    for c, lim in zip(reg_coord, rs):
        if not (0 <= c < lim):
            raise ValueError("register coordinate out of range")
    return tuple(t + r * ts for t, r, ts in zip(thread_coord, reg_coord, thread_shape))


def dot_thread_shape(logical_shape, max_threads=32):
    """Divisor pairs with product <= max_threads, largest by (product,
    smaller side, columns) -- the deterministic one-warp policy."""
    def divisors(n):
        return [d for d in range(1, n + 1) if n % d == 0]
    best = None
    for a in divisors(logical_shape[0]):
        for b in divisors(logical_shape[1]):
            if a * b <= max_threads:
                key = (a * b, min(a, b), b)
                if best is None or key > best[0]:
                    best = (key, (a, b))
    return best[1]


# --------------------------------------------------------------------------
# Triton LinearLayout: GF(2)-linear maps given by basis vectors
# --------------------------------------------------------------------------

def gf2_apply(bases, ins):
    """bases: {in_dim: [basis, ...]} with basis = tuple of out coordinates;
    ins: {in_dim: value}.  Each set bit i of an input selects basis i of that
    input dimension; the selected bases are XOR-ed coordinate by coordinate."""
    n_out = None
    for vecs in bases.values():
        for v in vecs:
            n_out = len(v)
            break
    out = [0] * (n_out or 0)
    for dim, val in ins.items():
        vecs = bases[dim]
        if val < 0 or val >= (1 << len(vecs)):
            raise ValueError(f"input {dim}={val} out of range")
        for i, v in enumerate(vecs):
            if (val >> i) & 1:
                out = [o ^ c for o, c in zip(out, v)]
    return tuple(out)


def _pack(vec, out_bits):
    """Concatenate the coordinates of an output vector into one integer."""
    word, shift = 0, 0
    for c, nb in zip(vec, out_bits):
        word |= c << shift
        shift += nb
    return word


def gf2_rank(bases, out_bits):
    """Rank over GF(2) of the matrix whose columns are all basis vectors,
    by Gaussian elimination on the packed words."""
    rows = [_pack(v, out_bits) for vecs in bases.values() for v in vecs]
    rank = 0
    for bit in range(sum(out_bits)):
        pivot = next((r for r in rows if (r >> bit) & 1), None)
        if pivot is None:
            continue
        rows.remove(pivot)
        rows = [r ^ pivot if (r >> bit) & 1 else r for r in rows]
        rank += 1
    return rank


def gf2_is_injective(bases, out_bits):
    return gf2_rank(bases, out_bits) == sum(len(v) for v in bases.values())


def gf2_is_surjective(bases, out_bits):
    return gf2_rank(bases, out_bits) == sum(out_bits)


# --------------------------------------------------------------------------
# The layout algebra ("Triton LinearLayout", sections "Combining layouts" and
# "invertAndCompose: derive data movement"), on flat maps: a map of nin input
# bits to nout output bits is (cols, nout) with cols[i] the packed output word
# of input bit i.
# --------------------------------------------------------------------------

def lin_apply(cols, x):
    """XOR of the columns selected by the set bits of x."""
    y = 0
    for i, c in enumerate(cols):
        if (x >> i) & 1:
            y ^= c
    return y


def lin_compose(outer, inner):
    """outer o inner: the page's rule -- outer applied to each basis of inner."""
    return [lin_apply(outer, c) for c in inner]


def lin_product(a, a_nout, b):
    """Direct sum: inputs of a then b, outputs of a then b (b's shifted up)."""
    return list(a) + [c << a_nout for c in b]


def lin_sublayout(cols, nout, in_bits, out_bits):
    """Keep the input bits listed in in_bits and the output bits listed in
    out_bits (each list in increasing order); kept output bits are packed."""
    out = []
    for i in in_bits:
        w = 0
        for k, b in enumerate(out_bits):
            w |= ((cols[i] >> b) & 1) << k
        out.append(w)
    return out


def lin_rank(cols, nout):
    rows = list(cols)
    rank = 0
    for bit in range(nout):
        pivot = next((r for r in rows if (r >> bit) & 1), None)
        if pivot is None:
            continue
        rows.remove(pivot)
        rows = [r ^ pivot if (r >> bit) & 1 else r for r in rows]
        rank += 1
    return rank


def lin_solve(S, nout, t):
    """A word q over S's input bits with lin_apply(S, q) == t, or None.

    Gauss-Jordan elimination on the augmented system [S | t]: each row is an
    output bit; the unknowns are S's input bits; free unknowns are set to 0."""
    nin = len(S)
    rows = []
    for b in range(nout):
        coef = 0
        for j, c in enumerate(S):
            if (c >> b) & 1:
                coef |= 1 << j
        rows.append([coef, (t >> b) & 1])
    pivots = []
    r = 0
    for j in range(nin):
        p = next((k for k in range(r, len(rows)) if (rows[k][0] >> j) & 1), None)
        if p is None:
            continue
        rows[r], rows[p] = rows[p], rows[r]
        for k in range(len(rows)):
            if k != r and (rows[k][0] >> j) & 1:
                rows[k] = [rows[k][0] ^ rows[r][0], rows[k][1] ^ rows[r][1]]
        pivots.append(j)
        r += 1
    if any(row[0] == 0 and row[1] for row in rows):
        return None
    q = 0
    for k, j in enumerate(pivots):
        if rows[k][1]:
            q |= 1 << j
    return q


def lin_invert_and_compose(R, S, nout):
    """Q with S(Q(x)) == R(x) for all x -- the page's S^-1 o R, where S may be
    non-injective (a pseudo-inverse) -- or None if R leaves S's image."""
    Q = []
    for c in R:
        q = lin_solve(S, nout, c)
        if q is None:
            return None
        Q.append(q)
    return Q


def log2_exact(n):
    if n <= 0 or n & (n - 1):
        raise ValueError(f"{n} is not a power of two")
    return n.bit_length() - 1


# --------------------------------------------------------------------------
# MI355X matrix-core fragments (v_mfma_f32_16x16x32_{f16,bf16})
# --------------------------------------------------------------------------
# One wave of 64 lanes.  Operand A (16 rows x 32 k): lane l holds row l % 16,
# k = 8*(l // 16) + e for its elements e = 0..7.  Operand B (32 k x 16 cols):
# lane l holds column l % 16 with the same k rule.  Result (16 x 16, fp32):
# lane l, register r holds row 4*(l // 16) + r, column l % 16.
# The k rule only has to agree between A and B: the instruction sums over the
# k slots, so any k order common to both operands gives the same sum.

def mfma16_a(lane, elem):
    return (lane % 16, 8 * (lane // 16) + elem)          # (row, k)


def mfma16_b(lane, elem):
    return (8 * (lane // 16) + elem, lane % 16)          # (k, col)


def mfma16_c(lane, reg):
    return (4 * (lane // 16) + reg, lane % 16)           # (row, col)


# v_mfma_f32_16x16x4_f32: operand A (16 rows x 4 k): lane l holds row l % 16,
# k = l // 16; operand B (4 k x 16 cols): column l % 16, same k; the result
# registers are those of the 16x16x32 shape (mfma16_c).

def mfma16f32_a(lane):
    return (lane % 16, lane // 16)                       # (row, k)


def mfma16f32_b(lane):
    return (lane // 16, lane % 16)                       # (k, col)


# v_mfma_f32_32x32x16_{f16,bf16}: operand 0 (32 rows x 16 k): lane l holds
# row l % 32, k = 8*(l // 32) + e; operand 1 (16 k x 32 cols): column l % 32,
# same k rule; result (32 x 32): lane l, register r holds row
# 8*(r // 4) + 4*(l // 32) + r % 4, column l % 32.

def mfma32_a(lane, elem):
    return (lane % 32, 8 * (lane // 32) + elem)


def mfma32_b(lane, elem):
    return (8 * (lane // 32) + elem, lane % 32)


def mfma32_c(lane, reg):
    return (8 * (reg // 4) + 4 * (lane // 32) + reg % 4, lane % 32)


# --------------------------------------------------------------------------
# The workgroup tile of the MI355X kernel
# --------------------------------------------------------------------------
# A tile config is (BM, BN, BK, WAVES_M, WAVES_N[, MF]), MF the fragment edge
# (16 or 32, default 16).  Wave w sits at wave row w // WAVES_N, wave column
# w % WAVES_N, and owns the sub-tile of WTM = BM / WAVES_M rows by
# WTN = BN / WAVES_N columns, made of (WTM/MF) x (WTN/MF) fragments.  The
# kernel feeds the B tile to the matrix core's row operand and the A tile to
# its column operand, so a fragment's result row is a C column and vice
# versa: within fragment (fm, fn), the value a lane's register holds at
# fragment position (i, j) is C(MF*fm + j, MF*fn + i).  The register index of
# that value is R*(fm*(WTN/MF) + fn) + r with R = MF*MF/64 registers per
# fragment.

def _cfg(cfg):
    BM, BN, BK, WM, WN = cfg[:5]
    MF = cfg[5] if len(cfg) > 5 else 16
    return BM, BN, BK, WM, WN, MF


def gemm_c_owner(cfg, reg, lane, wave):
    BM, BN, BK, WM, WN, MF = _cfg(cfg)
    WTM, WTN = BM // WM, BN // WN
    FN = WTN // MF
    R = MF * MF // 64
    r, f = reg % R, reg // R
    fm, fn = f // FN, f % FN
    frag_row, frag_col = (mfma16_c if MF == 16 else mfma32_c)(lane, r)
    row = (wave // WN) * WTM + MF * fm + frag_col
    col = (wave % WN) * WTN + MF * fn + frag_row
    return (row, col)


def gemm_regs_per_lane(cfg):
    BM, BN, BK, WM, WN, MF = _cfg(cfg)
    return (BM // WM) * (BN // WN) // 64


def gemm_c_bases(cfg):
    """The same ownership written as GF(2) bases {reg, lane, wave} -> (row, col)."""
    BM, BN, BK, WM, WN, MF = _cfg(cfg)
    WTM, WTN = BM // WM, BN // WN
    FM, FN = WTM // MF, WTN // MF
    if MF == 16:
        reg = [(0, 1), (0, 2)]
        lane = [(1, 0), (2, 0), (4, 0), (8, 0), (0, 4), (0, 8)]
    else:
        reg = [(0, 1), (0, 2), (0, 8), (0, 16)]
        lane = [(1, 0), (2, 0), (4, 0), (8, 0), (16, 0), (0, 4)]
    reg += [(0, MF << i) for i in range(log2_exact(FN))]
    reg += [(MF << i, 0) for i in range(log2_exact(FM))]
    wave = [(0, WTN << i) for i in range(log2_exact(WN))]
    wave += [(WTM << i, 0) for i in range(log2_exact(WM))]
    return {"reg": reg, "lane": lane, "wave": wave}


# --------------------------------------------------------------------------
# LDS operand tiles: 16-byte chunks, XOR swizzle
# --------------------------------------------------------------------------
# An operand tile has R rows (M rows for A, N rows for B) and G = BK/8 chunks
# of 8 consecutive k per row.  Chunk (r, g) lives in slot r*G + (g XOR s(r))
# with s(r) = ((r >> (3 - log2 G)) XOR (r >> 3)) mod G.

def lds_swizzle(r, G):
    shift = 3 - log2_exact(G)
    return ((r >> shift) ^ (r >> 3)) % G


def lds_slot(r, g, G):
    return r * G + (g ^ lds_swizzle(r, G))


def copy_kcontig(R, G, T, t, i):
    """Chunk moved by thread t at iteration i when the operand is stored with
    k contiguous: cooperative order (1, 0) over the (R, G) chunk grid.
    Returns (r, g) or None for an inactive tail lane."""
    lin = t + i * T
    if lin >= R * G:
        return None
    return coop_coordinate((R, G), (1, 0), lin)


def copy_mncontig(R, G, T, t, i):
    """8x8 block moved by thread t at iteration i when the operand is stored
    with rows (M or N) contiguous: cooperative order (0, 1) over the
    (R/8, G) grid of blocks.  Block (rb, g) covers rows 8rb..8rb+7 and
    k = 8g..8g+7.  Returns (rb, g) or None."""
    lin = t + i * T
    if lin >= (R // 8) * G:
        return None
    return coop_coordinate((R // 8, G), (0, 1), lin)


# --------------------------------------------------------------------------
# Direct-to-LDS tiles of the pipelined kernel (K step of 32)
# --------------------------------------------------------------------------
# k-contiguous operand [R rows][4 chunks of 8 k]: chunk (r, g) in slot
# 4r + (g XOR sk(r)), sk(r) = (bit1(r) XOR bit3(r)) + 2*bit2(r).
# Rows-contiguous operand [32 k rows][R/8 chunks of 8 rows]: chunk (k, c) in
# slot k*(R/8) + (c XOR sm(k)), sm(k) = 6*bit0(k) XOR 12*bit1(k) XOR
# 2*bit3(k).

def _bit(x, i):
    return (x >> i) & 1


def dma_kc_slot(r, g):
    sk = (_bit(r, 1) ^ _bit(r, 3)) + 2 * _bit(r, 2)
    return 4 * r + (g ^ sk)


def dma_mn_slot(R, k, c):
    """Slot of chunk c (8 rows) of k row k in a rows-contiguous operand tile of
    R rows.  With a multiple of 16 chunks per k row the chunk is XOR-ed with
    6*k0 ^ 12*k1 ^ 2*k3; with 24 chunks (R = 192) the XOR must stay inside
    aligned groups of 8 chunks: 6*k0 ^ 4*k1 ^ 2*k3."""
    if (R // 8) % 16 == 0:
        sm = (6 * _bit(k, 0)) ^ (12 * _bit(k, 1))
    else:
        sm = (6 * _bit(k, 0)) ^ (4 * _bit(k, 1))
    sm ^= 2 * _bit(k, 3)
    return k * (R // 8) + (c ^ sm)


# --------------------------------------------------------------------------
# The streaming tile for M <= 16 ([16, 64], 8 waves)
# --------------------------------------------------------------------------
# After the waves' partial tiles are summed, thread t = 64*wave + lane owns
# the two consecutive columns 2*(t % 32), 2*(t % 32) + 1 of row t // 32.

def skinny_c_owner(reg, lane, wave):
    t = 64 * wave + lane
    return (t // 32, 2 * (t % 32) + reg)
