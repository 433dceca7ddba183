"""Pins of the fp64 GEMM oracle against things other than itself.

Closed forms (identity, all-ones, zeros, rank one, permutation), brute force
against exact rational arithmetic, library routines for the number formats,
and storage equivalences.  Each is chosen so that a plausible mistake in the
oracle (a dropped term, a sign, a transposed operand or index, a wrong
epilogue order) fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import F16, BF16, F32


def f16_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16))


# ---- number formats -------------------------------------------------------------

def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, BF16)
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _edge_values(rng):
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        rng.uniform(-1, 1, 20000) * 2.0 ** -24,           # subnormal f16 range
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
                  2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 3.0e38, 3.5e38]),
    ])
    return x


def test_round_f16_matches_numpy():
    # numpy converts float64 -> float16 directly with round-half-to-even
    rng = np.random.default_rng(11)
    x = _edge_values(rng)
    got = oracle.round16(x, F16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_matches_torch_on_float32_inputs():
    # for values that are already float32, one RNE step is the whole story
    rng = np.random.default_rng(12)
    x = _edge_values(rng).astype(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.round16(x.astype(np.float64), BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_is_direct_from_fp64():
    # 1 + 2^-8 is a tie at bf16 precision (rounds to even 1.0); adding 2^-40
    # puts it above the tie, so it must round up.  A float32 detour would
    # erase the 2^-40 and round down.
    assert oracle.round16(np.array([1.0 + 2 ** -8 + 2 ** -40]), BF16)[0] == 0x3F81
    assert oracle.round16(np.array([1.0 + 2 ** -8]), BF16)[0] == 0x3F80
    assert oracle.round16(np.array([1.0 + 3 * 2 ** -8]), BF16)[0] == 0x3F82


def test_decode_f32_against_numpy():
    # every exponent field with random fractions, plus the special classes
    rng = np.random.default_rng(13)
    expo = np.repeat(np.arange(256, dtype=np.uint32), 512)
    frac = rng.integers(0, 1 << 23, expo.size, dtype=np.uint32)
    sign = rng.integers(0, 2, expo.size, dtype=np.uint32)
    bits = (sign << 31) | (expo << 23) | frac
    bits = np.concatenate([bits, np.array([0, 0x80000000, 1, 0x807FFFFF, 0x7F800000,
                                           0xFF800000, 0x7FC00000, 0x7F7FFFFF],
                                          dtype=np.uint32)])
    got = oracle.decode(bits, F32)
    ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_round_f32_matches_numpy():
    # numpy converts float64 -> float32 with round-half-to-even; the ties are
    # exact midpoints of neighbouring float32 values, including subnormals
    rng = np.random.default_rng(14)
    x = np.concatenate([
        rng.standard_normal(50000) * 10.0 ** rng.integers(-45, 39, 50000),
        rng.uniform(-1, 1, 20000) * 2.0 ** -126,
        np.array([0.0, -0.0, 3.4028234663852886e38, 3.4028235677973366e38, 1e39,
                  2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -151]),
    ])
    lo = rng.standard_normal(20000).astype(np.float32)
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    x = np.concatenate([x, mid])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    got = oracle.round_out(x, F32)
    assert np.array_equal(got, ref)


# ---- GEMM closed forms ----------------------------------------------------------

def gemm(M, N, K, A, B, lda=None, ldb=None, opA=0, opB=0, dt=F16, **kw):
    lda = lda or (M if opA else K)
    ldb = ldb or (K if opB else N)
    return oracle.gemm_block(M, N, K, A.reshape(-1), lda, opA, B.reshape(-1), ldb,
                             opB, dt, threads=2, **kw)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_identity_gives_a(dt):
    rng = np.random.default_rng(1)
    M, K = 7, 13
    a = rng.uniform(-2, 2, (M, K))
    A = f16_bits(a) if dt == F16 else oracle.round16(a, BF16)
    B = oracle.round16(np.eye(K), dt)
    C = gemm(M, K, K, A, B, dt=dt)
    assert np.array_equal(C, oracle.decode(A, dt).reshape(M, K))


def test_all_ones_gives_k():
    for M, N, K in [(1, 1, 1), (3, 5, 7), (16, 64, 32), (2, 3, 1000)]:
        A = f16_bits(np.ones((M, K)))
        B = f16_bits(np.ones((K, N)))
        assert np.array_equal(gemm(M, N, K, A, B), np.full((M, N), float(K)))


def test_zeros_give_zero():
    rng = np.random.default_rng(2)
    A = f16_bits(rng.uniform(-1, 1, (5, 9)))
    B = f16_bits(np.zeros((9, 4)))
    assert np.array_equal(gemm(5, 4, 9, A, B), np.zeros((5, 4)))


def test_rank_one_closed_form():
    # A = u 1^T, B = 1 v^T  =>  C = K u v^T, exactly for these dyadic values
    u = np.array([0.5, -1.0, 2.0, 0.25, -3.0])
    v = np.array([1.0, -0.5, 0.125, 4.0])
    K = 6
    A = f16_bits(np.outer(u, np.ones(K)))
    B = f16_bits(np.outer(np.ones(K), v))
    assert np.array_equal(gemm(5, 4, K, A, B), K * np.outer(u, v))


def test_permutation_permutes_columns():
    # non-square shapes: a transposed operand or swapped index cannot pass
    rng = np.random.default_rng(3)
    M, K = 4, 6
    a = rng.uniform(-1, 1, (M, K))
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0        # column j of A.P is column perm[j] of A
    A = f16_bits(a)
    C = gemm(M, K, K, A, f16_bits(P))
    assert np.array_equal(C, oracle.decode(A, F16).reshape(M, K)[:, perm])


def _exact_sum(a, b):
    M, K = a.shape
    N = b.shape[1]
    return [[sum(Fraction(float(a[m, k])) * Fraction(float(b[k, n])) for k in range(K))
             for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("dt", [F16, BF16])
def test_brute_force_exact(dt):
    rng = np.random.default_rng(4)
    for M, N, K in [(1, 1, 1), (2, 3, 5), (5, 4, 3), (3, 7, 11)]:
        A = oracle.round16(rng.uniform(-3, 3, (M, K)), dt)
        B = oracle.round16(rng.uniform(-3, 3, (K, N)), dt)
        a = oracle.decode(A, dt).reshape(M, K)
        b = oracle.decode(B, dt).reshape(K, N)
        exact = _exact_sum(a, b)
        C = gemm(M, N, K, A, B, dt=dt)
        for m in range(M):
            for n in range(N):
                bound = K * 2.0 ** -53 * sum(abs(a[m, k] * b[k, n]) for k in range(K))
                assert abs(Fraction(C[m, n]) - exact[m][n]) <= Fraction(bound)


def test_against_numpy_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 33, 47, 129
    A = f16_bits(rng.standard_normal((M, K)))
    B = f16_bits(rng.standard_normal((K, N)))
    a = oracle.decode(A, F16).reshape(M, K)
    b = oracle.decode(B, F16).reshape(K, N)
    ref = a @ b
    bound = 2 * K * 2.0 ** -53 * (np.abs(a) @ np.abs(b))
    assert np.all(np.abs(gemm(M, N, K, A, B) - ref) <= bound)


# ---- storage: transposes, leading dimensions, sub-blocks ------------------------

def test_transposed_storage_is_bit_identical():
    rng = np.random.default_rng(6)
    M, N, K = 9, 10, 21
    a = f16_bits(rng.uniform(-1, 1, (M, K))).reshape(M, K)
    b = f16_bits(rng.uniform(-1, 1, (K, N))).reshape(K, N)
    ref = gemm(M, N, K, a, b)
    # A^T stored [K][lda] with padding, B^T stored [N][ldb] with padding
    lda, ldb = M + 3, K + 5
    at = np.full((K, lda), 0x7E00, dtype=np.uint16)
    at[:, :M] = a.T
    bt = np.full((N, ldb), 0x7E00, dtype=np.uint16)
    bt[:, :K] = b.T
    got = oracle.gemm_block(M, N, K, at.reshape(-1), lda, 1, bt.reshape(-1), ldb, 1, F16)
    assert np.array_equal(got, ref)
    got = oracle.gemm_block(M, N, K, at.reshape(-1), lda, 1, b.reshape(-1), N, 0, F16)
    assert np.array_equal(got, ref)


def test_padding_never_read():
    # NaN in the leading-dimension padding must not reach the result
    rng = np.random.default_rng(7)
    M, N, K = 6, 5, 4
    a = f16_bits(rng.uniform(-1, 1, (M, K))).reshape(M, K)
    b = f16_bits(rng.uniform(-1, 1, (K, N))).reshape(K, N)
    A = np.full((M, K + 4), 0x7E00, dtype=np.uint16)
    A[:, :K] = a
    B = np.full((K, N + 2), 0x7E00, dtype=np.uint16)
    B[:, :N] = b
    got = oracle.gemm_block(M, N, K, A.reshape(-1), K + 4, 0, B.reshape(-1), N + 2, 0, F16)
    assert np.isfinite(got).all()
    assert np.array_equal(got, gemm(M, N, K, a, b))


def test_blocks_and_cells_agree_with_full():
    rng = np.random.default_rng(8)
    M, N, K = 20, 17, 40
    A = f16_bits(rng.uniform(-1, 1, (M, K)))
    B = f16_bits(rng.uniform(-1, 1, (K, N)))
    full = gemm(M, N, K, A, B)
    blk = oracle.gemm_block(M, N, K, A, K, 0, B, N, 0, F16, m_range=(3, 11), n_range=(5, 16))
    assert np.array_equal(blk, full[3:11, 5:16])
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    cells = oracle.gemm_cells(M, N, K, A, K, 0, B, N, 0, F16, ms, ns)
    assert np.array_equal(cells, full[ms, ns])
    one = oracle.gemm_block(M, N, K, A, K, 0, B, N, 0, F16, threads=1)
    assert np.array_equal(one, full)


# ---- epilogue ---------------------------------------------------------------------

def test_epilogue_closed_forms():
    rng = np.random.default_rng(9)
    M, N, K = 5, 6, 3
    A = f16_bits(rng.uniform(-1, 1, (M, K)))
    Z = f16_bits(np.zeros((K, N)))
    bias = f16_bits(rng.uniform(-2, 2, N))
    R = f16_bits(rng.uniform(-2, 2, (M, N)))
    bv = oracle.decode(bias, F16)
    rv = oracle.decode(R, F16).reshape(M, N)
    # B = 0: acc = 0, so C = relu(bias) + R
    C = gemm(M, N, K, A, Z, bias=bias, relu=True, R=R, ldr=N)
    assert np.array_equal(C, np.maximum(bv, 0)[None, :] + rv)
    C = gemm(M, N, K, A, Z, bias=bias)
    assert np.array_equal(C, np.broadcast_to(bv, (M, N)))
    C = gemm(M, N, K, A, Z, R=R, ldr=N)
    assert np.array_equal(C, rv)


def test_epilogue_order_relu_before_residual():
    # acc = -1 everywhere (A = 1, B = -1, K = 1), bias 0.5, residual 0.25
    # relu(acc + bias) + R = 0 + 0.25; R before relu would give 0; relu
    # before bias would give 0.75
    A = f16_bits(np.ones((2, 1)))
    B = f16_bits(-np.ones((1, 3)))
    bias = f16_bits(np.full(3, 0.5))
    R = f16_bits(np.full((2, 3), 0.25))
    C = gemm(2, 3, 1, A, B, bias=bias, relu=True, R=R, ldr=3)
    assert np.array_equal(C, np.full((2, 3), 0.25))
    C = gemm(2, 3, 1, A, B, relu=True)
    assert np.array_equal(C, np.zeros((2, 3)))
    C = gemm(2, 3, 1, A, B)
    assert np.array_equal(C, -np.ones((2, 3)))


def test_residual_leading_dimension():
    M, N, K = 3, 4, 2
    A = f16_bits(np.zeros((M, K)))
    B = f16_bits(np.zeros((K, N)))
    ldr = 7
    R = np.full((M, ldr), 0x7E00, dtype=np.uint16)
    r = np.arange(M * N, dtype=np.float64).reshape(M, N)
    R[:, :N] = f16_bits(r).reshape(M, N)
    C = gemm(M, N, K, A, B, R=R.reshape(-1), ldr=ldr)
    assert np.array_equal(C, r)


def test_accept_rule():
    Cref = np.array([[1.0, -2.0], [100.0, 0.0]])
    bits = oracle.round16(Cref, F16).reshape(2, 2)
    rep = oracle.accept(bits, Cref, F16)
    assert rep["ok"] and rep["bit_match"] == 1.0
    bad = bits.copy()
    bad[1, 0] = oracle.round16(np.array([102.0]), F16)[0]   # error 2 > 0.01 + 1.0
    assert not oracle.accept(bad, Cref, F16)["ok"]
    nan = bits.copy()
    nan[0, 0] = 0x7E00
    assert not oracle.accept(nan, Cref, F16)["ok"]


# ---- row scale and output dtypes ------------------------------------------------
# "Named layouts" (NineToothed), section "Contract": a row scale is the
# broadcast operand of axes "m"; the epilogue is relu(acc * scale + bias) + R.

def test_row_scale_identity_closed_form():
    rng = np.random.default_rng(21)
    M, K = 6, 5
    A = f16_bits(rng.uniform(-2, 2, (M, K)))
    I = f16_bits(np.eye(K))
    s = f16_bits(rng.uniform(-3, 3, M))
    a = oracle.decode(A, F16).reshape(M, K)
    sv = oracle.decode(s, F16)
    C = gemm(M, K, K, A, I, scale=s)
    assert np.array_equal(C, sv[:, None] * a)
    bias = f16_bits(rng.uniform(-2, 2, K))
    R = f16_bits(rng.uniform(-2, 2, (M, K)))
    C = gemm(M, K, K, A, I, scale=s, bias=bias, relu=True, R=R, ldr=K)
    exp = np.maximum(sv[:, None] * a + oracle.decode(bias, F16)[None, :], 0) + \
        oracle.decode(R, F16).reshape(M, K)
    assert np.array_equal(C, exp)


def test_row_scale_applies_before_bias():
    # acc = 2 (K = 1), scale 3, bias -5: scale then bias gives 1; bias then
    # scale would give -9 (0 after ReLU); scale after ReLU would give 0
    A = f16_bits(np.full((2, 1), 2.0))
    B = f16_bits(np.ones((1, 3)))
    s = f16_bits(np.full(2, 3.0))
    bias = f16_bits(np.full(3, -5.0))
    C = gemm(2, 3, 1, A, B, scale=s, bias=bias, relu=True)
    assert np.array_equal(C, np.ones((2, 3)))


def test_row_scale_all_ones_gives_k_times_scale():
    M, N, K = 4, 3, 9
    s = f16_bits(np.array([1.0, -2.0, 0.5, 0.0]))
    C = gemm(M, N, K, f16_bits(np.ones((M, K))), f16_bits(np.ones((K, N))), scale=s)
    assert np.array_equal(C, np.array([9.0, -18.0, 4.5, 0.0])[:, None] * np.ones((M, N)))


@pytest.mark.parametrize("in_dt,out_dt", [(F16, BF16), (BF16, F16), (F16, F32), (BF16, F32)])
def test_brute_force_exact_with_scale_and_mixed_dtypes(in_dt, out_dt):
    rng = np.random.default_rng(22)
    M, N, K = 3, 5, 7
    A = oracle.round16(rng.uniform(-3, 3, (M, K)), in_dt)
    B = oracle.round16(rng.uniform(-3, 3, (K, N)), in_dt)
    s = oracle.round_out(rng.uniform(-2, 2, M), out_dt)
    bias = oracle.round_out(rng.uniform(-2, 2, N), out_dt)
    R = oracle.round_out(rng.uniform(-2, 2, (M, N)), out_dt).reshape(-1)
    a = oracle.decode(A, in_dt).reshape(M, K)
    b = oracle.decode(B, in_dt).reshape(K, N)
    sv, bv = oracle.decode(s, out_dt), oracle.decode(bias, out_dt)
    rv = oracle.decode(R, out_dt).reshape(M, N)
    exact = _exact_sum(a, b)
    C = gemm(M, N, K, A, B, dt=in_dt, out_dtype=out_dt, scale=s, bias=bias, R=R, ldr=N)
    for m in range(M):
        for n in range(N):
            e = exact[m][n] * Fraction(sv[m]) + Fraction(bv[n]) + Fraction(rv[m, n])
            bound = 4 * K * 2.0 ** -53 * (abs(sv[m]) * sum(abs(a[m, k] * b[k, n]) for k in range(K))
                                          + abs(bv[n]) + abs(rv[m, n]))
            assert abs(Fraction(C[m, n]) - e) <= Fraction(bound)


def test_f32_epilogue_operands_are_read_as_binary32():
    # a value only binary32 can hold (1 + 2^-20) must survive as is
    v = np.array([1.0 + 2.0 ** -20], dtype=np.float32)
    bias = np.ascontiguousarray(np.repeat(v, 2).view(np.uint32))
    C = gemm(1, 2, 1, f16_bits(np.zeros((1, 1))), f16_bits(np.zeros((1, 2))),
             out_dtype=F32, bias=bias)
    assert np.array_equal(C, np.full((1, 2), 1.0 + 2.0 ** -20))


def test_accept_rule_f32_output():
    Cref = np.array([[1.0 + 2.0 ** -30, -2.0], [100.0, 0.0]])
    bits = oracle.round_out(Cref, F32)
    rep = oracle.accept(bits, Cref, F32)
    assert rep["ok"] and rep["bit_match"] == 1.0
    bad = bits.copy()
    bad[1, 0] = np.array([102.0], dtype=np.float32).view(np.uint32)[0]
    assert not oracle.accept(bad, Cref, F32)["ok"]
    nan = bits.copy()
    nan[0, 0] = 0x7FC00000
    assert not oracle.accept(nan, Cref, F32)["ok"]


# ---- binary32 inputs ------------------------------------------------------------

def f32_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32).view(np.uint32))


def test_f32_inputs_identity_and_ones():
    rng = np.random.default_rng(23)
    A = rng.standard_normal((5, 7)).astype(np.float32)
    C = gemm(5, 7, 7, f32_bits(A), f32_bits(np.eye(7)), dt=F32, out_dtype=F32)
    assert np.array_equal(C, A.astype(np.float64))
    C = gemm(3, 4, 11, f32_bits(np.ones((3, 11))), f32_bits(np.ones((11, 4))), dt=F32)
    assert np.array_equal(C, np.full((3, 4), 11.0))


def test_f32_inputs_brute_force():
    rng = np.random.default_rng(24)
    M, N, K = 4, 5, 9
    a = rng.uniform(-3, 3, (M, K)).astype(np.float32)
    b = rng.uniform(-3, 3, (K, N)).astype(np.float32)
    C = gemm(M, N, K, f32_bits(a), f32_bits(b), dt=F32, out_dtype=F32)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(a[m, k])) * Fraction(float(b[k, n])) for k in range(K))
            # each binary32 product is exact in fp64 up to its 48-bit width; K additions
            bound = 2 * K * 2.0 ** -53 * sum(abs(float(a[m, k]) * float(b[k, n])) for k in range(K))
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(bound)


def test_f32_transposed_storage_bit_identical():
    rng = np.random.default_rng(25)
    a = rng.standard_normal((6, 8)).astype(np.float32)
    b = rng.standard_normal((8, 5)).astype(np.float32)
    base = gemm(6, 5, 8, f32_bits(a), f32_bits(b), dt=F32, out_dtype=F32)
    t = gemm(6, 5, 8, f32_bits(a.T.copy()), f32_bits(b.T.copy()), opA=1, opB=1, dt=F32,
             out_dtype=F32)
    assert np.array_equal(base, t)
