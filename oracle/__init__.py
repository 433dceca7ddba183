"""The oracle: plain, slow, obviously correct CPU implementations.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
and the CPU-baseline leg of bench.py may import anything from this package.
It shares no code with the HIP library (thread_register_tile_amd) and never
imports it.

* gemm_block / gemm_cells -- the fp64 GEMM + epilogue in plain C
  (gemm_ref.c), reached through ctypes.
* decode / round16 -- the 16-bit float formats from their definitions.
* layout_ref -- the ownership, copy and swizzle maps in plain Python ints.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16 = 1
BF16 = 2

_lib = None


def lib():
    """Load oracle/_liborc.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_decode_f16.restype = ctypes.c_double
        L.orc_decode_f16.argtypes = [ctypes.c_uint16]
        L.orc_decode_bf16.restype = ctypes.c_double
        L.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        L.orc_round_f16.restype = ctypes.c_uint16
        L.orc_round_f16.argtypes = [ctypes.c_double]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_round_array.restype = None
        L.orc_round_array.argtypes = [vp, vp, i64, i32]
        L.orc_decode_array.restype = None
        L.orc_decode_array.argtypes = [vp, vp, i64, i32]
        L.orc_gemm_block.restype = i32
        L.orc_gemm_block.argtypes = [i64, i64, i64, vp, i64, i32, vp, i64, i32,
                                     i32, vp, i32, vp, i64, i32,
                                     i64, i64, i64, i64, vp, i32]
        L.orc_gemm_cells.restype = i32
        L.orc_gemm_cells.argtypes = [i64, i64, i64, vp, i64, i32, vp, i64, i32,
                                     i32, vp, i32, vp, i64, i32,
                                     vp, vp, i64, vp, i32]
        L.orc_max_threads.restype = i32
        L.orc_max_threads.argtypes = []
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a, name):
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.dtype == np.uint16 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous numpy uint16 array of raw bits")
    return a


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Decode raw 16-bit patterns (uint16) to float64, from the format definition."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().orc_decode_array(_ptr(b), _ptr(out), b.size, dtype)
    return out


def round16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to 16-bit patterns, to nearest with ties to even."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_round_array(_ptr(v), _ptr(out), v.size, dtype)
    return out


def gemm_block(M, N, K, A, lda, opA, B, ldb, opB, in_dtype, bias=None,
               relu=False, R=None, ldr=0, epi_dtype=None,
               m_range=None, n_range=None, threads=None) -> np.ndarray:
    """fp64 reference of the block m_range x n_range of epilogue(A.B).

    A, B, bias, R are flat uint16 buffers of raw bits addressed exactly as the
    library addresses them (leading dimensions in elements, explicit op flags).
    Returns an (m_hi-m_lo, n_hi-n_lo) float64 array, unrounded.
    """
    A = _u16(A, "A"); B = _u16(B, "B"); bias = _u16(bias, "bias"); R = _u16(R, "R")
    m_lo, m_hi = m_range if m_range is not None else (0, M)
    n_lo, n_hi = n_range if n_range is not None else (0, N)
    out = np.empty((m_hi - m_lo, n_hi - n_lo), dtype=np.float64)
    rc = lib().orc_gemm_block(M, N, K, _ptr(A), lda, int(opA), _ptr(B), ldb,
                              int(opB), in_dtype, _ptr(bias), int(bool(relu)),
                              _ptr(R), ldr, epi_dtype or in_dtype,
                              m_lo, m_hi, n_lo, n_hi, _ptr(out),
                              threads or default_threads())
    if rc != 0:
        raise ValueError("oracle gemm_block: bad arguments")
    return out


def gemm_cells(M, N, K, A, lda, opA, B, ldb, opB, in_dtype, ms, ns, bias=None,
               relu=False, R=None, ldr=0, epi_dtype=None, threads=None) -> np.ndarray:
    """fp64 reference of the scattered cells (ms[i], ns[i]), one by one."""
    A = _u16(A, "A"); B = _u16(B, "B"); bias = _u16(bias, "bias"); R = _u16(R, "R")
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    rc = lib().orc_gemm_cells(M, N, K, _ptr(A), lda, int(opA), _ptr(B), ldb,
                              int(opB), in_dtype, _ptr(bias), int(bool(relu)),
                              _ptr(R), ldr, epi_dtype or in_dtype,
                              _ptr(ms), _ptr(ns), ms.size, _ptr(out),
                              threads or default_threads())
    if rc != 0:
        raise ValueError("oracle gemm_cells: bad arguments")
    return out


def accept(C_bits: np.ndarray, Cref: np.ndarray, out_dtype: int,
           atol: float = 1e-2, rtol: float = 1e-2) -> dict:
    """The acceptance rule: every cell |C - Cref| <= atol + rtol*|Cref|, no NaN/Inf.

    Cref is the unrounded fp64 reference.  Returns diagnostics (max errors,
    relative Frobenius error, fraction of cells bit-equal to the RNE-rounded
    reference) next to the pass/fail verdict.
    """
    C = decode(C_bits, out_dtype)
    err = np.abs(C - Cref)
    finite = np.isfinite(C)
    bound = atol + rtol * np.abs(Cref)
    ok = bool(finite.all() and (err <= bound).all())
    ref16 = round16(Cref, out_dtype)
    den = np.linalg.norm(Cref)
    return {
        "ok": ok,
        "n": int(C.size),
        "violations": int((~finite).sum() + (finite & (err > bound)).sum()),
        "max_abs": float(np.nanmax(err)) if C.size else 0.0,
        "max_rel": float(np.nanmax(err / np.maximum(np.abs(Cref), 1e-30))) if C.size else 0.0,
        "frob_rel": float(np.linalg.norm(np.nan_to_num(C - Cref)) / den) if den > 0 else 0.0,
        "bit_match": float((np.asarray(C_bits, dtype=np.uint16) == ref16).mean()) if C.size else 1.0,
    }
