"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only names the workloads
(shapes, strides, storage order, value distribution, epilogue flags) and
draws their raw 16-bit operand buffers from a seeded generator.  Both the
oracle and the HIP path are fed these same bytes.

Recipe (one generator per tensor): numpy PCG64 seeded with
[config_seed, tensor_id]; tensor ids A=0, B=1, bias=2, residual=3, row
scale=4.  Values are drawn in float64 in *storage* order (A^T order when A is
stored transposed), rounded to the element type (float16: numpy's
float64->float16 conversion; bfloat16: float64->float32, then
round-to-nearest-even on the float32 bits; float32: numpy's float64->float32
conversion) and written into a padded buffer whose leading-dimension padding
holds NaN, so that any read of the padding poisons the result.  A leading
dimension below the row length (rows that overlap in memory) draws the
operand's whole extent, (rows - 1)*ld + cols values, as one row.  A and B use
the input type; bias, residual and row scale use the output type.
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

F16 = 1
BF16 = 2
F32 = 3                 # binary32
DTYPE_NAMES = {F16: "f16", BF16: "bf16", F32: "f32"}
ELEM_BYTES = {F16: 2, BF16: 2, F32: 4}

TENSOR_A, TENSOR_B, TENSOR_BIAS, TENSOR_R, TENSOR_SCALE = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    opA: int = 0            # 0: A stored [M][lda], 1: A stored as A^T [K][lda]
    opB: int = 0            # 0: B stored [K][ldb], 1: B stored as B^T [N][ldb]
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    ldr: Optional[int] = None     # residual leading dimension; None: N
    dtype: int = F16       # input type of A and B (F16, BF16 or F32)
    out_dtype: Optional[int] = None   # output type (C, bias, residual, row scale); None: dtype
    row_scale: bool = False
    bias: bool = False
    relu: bool = False
    residual: bool = False
    dist: str = "uniform"   # uniform | normal | ternary (exact-arithmetic mode)
    scale: float = 1.0      # half-width for uniform, divisor for normal
    seed: int = 0
    tile: Optional[tuple] = None  # explicit (BM, BN, BK) tile, or None
    regtile: Optional[tuple] = None  # (lm, ln, max_threads): the vector-lane register-tile GEMM

    @property
    def a_rows(self):
        return self.K if self.opA else self.M

    @property
    def a_cols(self):
        return self.M if self.opA else self.K

    @property
    def b_rows(self):
        return self.N if self.opB else self.K

    @property
    def b_cols(self):
        return self.K if self.opB else self.N

    @property
    def lda_(self):
        return self.lda if self.lda is not None else self.a_cols

    @property
    def ldb_(self):
        return self.ldb if self.ldb is not None else self.b_cols

    @property
    def ldc_(self):
        return self.ldc if self.ldc is not None else self.N

    @property
    def ldr_(self):
        return self.ldr if self.ldr is not None else self.N

    @property
    def odt(self):
        return self.out_dtype if self.out_dtype is not None else self.dtype

    @property
    def flops(self):
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self):
        o = ELEM_BYTES[self.odt]
        b = ELEM_BYTES[self.dtype] * (self.M * self.K + self.K * self.N) + o * self.M * self.N
        if self.bias:
            b += o * self.N
        if self.residual:
            b += o * self.M * self.N
        if self.row_scale:
            b += o * self.M
        return b


# The five GEMM workloads shaped like the pages' examples: a tiny tile, a square
# 4096^3 GEMM, a GEMM with bias, ReLU and residual, a transposed, ragged and
# padded GEMM, and a skinny memory-bound GEMM.
TINY = Workload("tiny", 64, 64, 32, dtype=F16, dist="uniform", scale=1.0,
                seed=1, tile=(16, 64, 32))
SQUARE = Workload("square", 4096, 4096, 4096, dtype=F16, dist="normal",
                  scale=8.0, seed=2)
EPILOGUE = Workload("epilogue", 8192, 8192, 4096, dtype=BF16, bias=True,
                    relu=True, residual=True, dist="uniform", scale=1.0, seed=3)
RAGGED = Workload("ragged", 4000, 3072, 5000, opA=1, lda=5064, ldb=3136,
                  dtype=F16, dist="uniform", scale=0.5, seed=4)
SKINNY = Workload("skinny", 16, 16384, 16384, dtype=F16, dist="normal",
                  scale=128.0, seed=5)

# A further epilogue variant: the epilogue shape with bf16 inputs, a binary32
# output and binary32 epilogue operands, and a row scale ("Named layouts",
# section "Contract": the axes-"m" broadcast operand).
ROWSCALE = Workload("rowscale", 8192, 8192, 4096, dtype=BF16, out_dtype=F32, row_scale=True,
                    bias=True, relu=True, residual=True, dist="uniform", scale=1.0, seed=6)

# The square shape with binary32 operands and output: the register-tile dot
# of "My Triton From Scratch, Part 16: Register Tiles" computes in f32
# throughout (section "What Version 16 does not optimize").
F32SQUARE = Workload("f32square", 4096, 4096, 4096, dtype=F32, dist="normal", scale=8.0, seed=8)

# The same shape on general-purpose vector lanes with a 64x64 register tile
# (thread shape (8, 8), registers (8, 8)): the execution model of "My Triton
# From Scratch, Part 16: Register Tiles", section "Register-valued
# loop-carried accumulators", without the matrix cores.
REGTILE = Workload("regtile", 4096, 4096, 4096, dtype=F32, dist="normal", scale=8.0, seed=9,
                   regtile=(64, 64, 64))

CONFIGS = {w.name: w for w in (TINY, SQUARE, EPILOGUE, RAGGED, SKINNY, ROWSCALE, F32SQUARE,
                               REGTILE)}


def shrink(w: Workload, M=None, N=None, K=None, **kw) -> Workload:
    """A smaller workload with the same storage scheme, dtype, epilogue and
    distribution; leading dimensions keep the same padding beyond the
    contiguous extent as the original."""
    M = M or w.M
    N = N or w.N
    K = K or w.K
    new = replace(w, M=M, N=N, K=K, lda=None, ldb=None, ldc=None, ldr=None, **kw)
    pad_a = (w.lda_ - w.a_cols) if w.lda is not None else 0
    pad_b = (w.ldb_ - w.b_cols) if w.ldb is not None else 0
    return replace(new, lda=new.a_cols + pad_a if pad_a else None,
                   ldb=new.b_cols + pad_b if pad_b else None)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, to nearest with ties to even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def to_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    """Raw bits of x rounded to dtype: uint16, or uint32 for F32."""
    if dtype == F16:
        return np.ascontiguousarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


NAN_BITS = {F16: np.uint16(0x7E00), BF16: np.uint16(0x7FC0), F32: np.uint32(0x7FC00000)}


def _draw(w: Workload, tensor_id: int, rows: int, cols: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, tensor_id])
    shape = (rows, cols)
    if w.dist == "uniform":
        x = rng.uniform(-w.scale, w.scale, size=shape)
    elif w.dist == "normal":
        x = rng.standard_normal(size=shape) / w.scale
    elif w.dist == "ternary":
        # exact-arithmetic mode: operands in {-1, 0, 1}, epilogue terms in {-2..2}
        lim = 2 if tensor_id in (TENSOR_BIAS, TENSOR_R, TENSOR_SCALE) else 1
        x = rng.integers(-lim, lim + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(w.dist)
    return x


def _padded(w: Workload, tensor_id: int, rows: int, cols: int, ld: int, dtype=None) -> np.ndarray:
    dtype = dtype or w.dtype
    if ld < cols:
        # overlapping rows (a positive stride below the row length): element
        # (r, c) sits at r*ld + c, so the buffer is the operand's extent,
        # drawn as one row of (rows - 1)*ld + cols values
        return to_bits(_draw(w, tensor_id, 1, (rows - 1) * ld + cols), dtype).reshape(-1)
    bits = to_bits(_draw(w, tensor_id, rows, cols), dtype)
    buf = np.full((rows, ld), NAN_BITS[dtype], dtype=bits.dtype)
    buf[:, :cols] = bits
    return buf.reshape(-1)


def make_inputs(w: Workload) -> dict:
    """Raw host buffers for a workload: A, B (flat raw bits of the input type)
    and, if enabled, bias [N], residual [M, N] (leading dimension ldr_) and row
    scale [M] (flat, of the output type: uint16, or uint32 for F32)."""
    out = {
        "A": _padded(w, TENSOR_A, w.a_rows, w.a_cols, w.lda_),
        "B": _padded(w, TENSOR_B, w.b_rows, w.b_cols, w.ldb_),
        "bias": None,
        "R": None,
        "scale": None,
    }
    if w.bias:
        out["bias"] = _padded(w, TENSOR_BIAS, 1, w.N, w.N, w.odt)
    if w.residual:
        out["R"] = _padded(w, TENSOR_R, w.M, w.N, w.ldr_, w.odt)
    if w.row_scale:
        out["scale"] = _padded(w, TENSOR_SCALE, 1, w.M, w.M, w.odt)
    return out


# ---- the rank-1 block reduction ("My Triton From Scratch, Part 12: CUDA Tile
# Layouts", section "Output shape is not always thread shape") -------------------

@dataclass(frozen=True)
class ReduceWorkload:
    name: str
    n: int
    block: int
    dtype: int = F16
    op: int = 0             # 0 sum, 1 max, 2 min
    dist: str = "normal"    # normal | uniform | ternary (exact sums)
    scale: float = 1.0
    seed: int = 0

    @property
    def nblocks(self):
        return -(-self.n // self.block)

    @property
    def algorithmic_bytes(self):
        return ELEM_BYTES[self.dtype] * self.n + 4 * self.nblocks


REDUCE = ReduceWorkload("reduce", 1 << 28, 1024, dtype=F16, op=0, dist="normal", scale=1.0, seed=7)


def make_reduce_input(w: ReduceWorkload) -> np.ndarray:
    """The n input elements (raw bits: uint16, or uint32 for F32), tensor id 0."""
    rng = np.random.default_rng([w.seed, 0])
    if w.dist == "normal":
        x = rng.standard_normal(w.n) / w.scale
    elif w.dist == "uniform":
        x = rng.uniform(-w.scale, w.scale, w.n)
    elif w.dist == "ternary":
        x = rng.integers(-1, 2, w.n).astype(np.float64)
    else:
        raise ValueError(w.dist)
    return to_bits(x, w.dtype)
