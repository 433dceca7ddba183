"""The oracle: plain, slow, obviously correct CPU implementations.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
and the CPU-baseline leg of bench.py may import anything from this package.
It shares no code with the HIP library (thread_register_tile_amd) and never
imports it.

* gemm_block / gemm_cells -- the fp64 GEMM + epilogue in plain C
  (gemm_ref.c), reached through ctypes.
* decode / round16 / round_out -- the binary16, bfloat16 and binary32
  formats from their definitions.
* layout_ref -- the ownership, copy and swizzle maps in plain Python ints,
  and the GF(2) layout algebra.
* reduce_ref -- the rank-1 block reduction (sum / max / min per block).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16 = 1
BF16 = 2
F32 = 3          # binary32: inputs, outputs, epilogue operands

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
        L.orc_decode_f32.restype = ctypes.c_double
        L.orc_decode_f32.argtypes = [ctypes.c_uint32]
        L.orc_round_f32.restype = ctypes.c_uint32
        L.orc_round_f32.argtypes = [ctypes.c_double]
        L.orc_round_array.restype = None
        L.orc_round_array.argtypes = [vp, vp, i64, i32]
        L.orc_decode_array.restype = None
        L.orc_decode_array.argtypes = [vp, vp, i64, i32]
        L.orc_gemm_block.restype = i32
        L.orc_gemm_block.argtypes = [i64, i64, i64, vp, i64, i32, vp, i64, i32,
                                     i32, vp, vp, i32, vp, i64, i32,
                                     i64, i64, i64, i64, vp, i32]
        L.orc_gemm_cells.restype = i32
        L.orc_gemm_cells.argtypes = [i64, i64, i64, vp, i64, i32, vp, i64, i32,
                                     i32, vp, vp, i32, vp, i64, i32,
                                     vp, vp, i64, vp, i32]
        L.orc_max_threads.restype = i32
        L.orc_max_threads.argtypes = []
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits_type(dtype):
    return np.uint32 if dtype == F32 else np.uint16


def _u16(a, name):
    return _raw(a, name, F16)


def _raw(a, name, dtype):
    """Validate a flat buffer of raw bit patterns of `dtype` (uint16, or
    uint32 for binary32)."""
    if a is None:
        return None
    t = _bits_type(dtype)
    if not (isinstance(a, np.ndarray) and a.dtype == t and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous numpy {t.__name__} array of raw bits")
    return a


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Decode raw bit patterns (uint16; uint32 for F32) to float64, from the
    format definition."""
    b = np.ascontiguousarray(bits, dtype=_bits_type(dtype))
    out = np.empty(b.shape, dtype=np.float64)
    lib().orc_decode_array(_ptr(b), _ptr(out), b.size, dtype)
    return out


def round_out(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to `dtype` bit patterns (uint16, or uint32 for
    F32), to nearest with ties to even."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=_bits_type(dtype))
    lib().orc_round_array(_ptr(v), _ptr(out), v.size, dtype)
    return out


def round16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to 16-bit patterns, to nearest with ties to even."""
    if dtype == F32:
        raise ValueError("round16 takes a 16-bit dtype")
    return round_out(x, dtype)


def gemm_block(M, N, K, A, lda, opA, B, ldb, opB, in_dtype, bias=None,
               relu=False, R=None, ldr=0, out_dtype=None, scale=None,
               m_range=None, n_range=None, threads=None) -> np.ndarray:
    """fp64 reference of the block m_range x n_range of epilogue(A.B).

    A, B are flat buffers of raw bits of `in_dtype` (uint16, or uint32 for
    F32); scale [M], bias
    [N] and R are flat buffers of raw bits of the output dtype (uint32 for
    F32), addressed exactly as the library addresses them (leading
    dimensions in elements, explicit op flags).  Returns an
    (m_hi-m_lo, n_hi-n_lo) float64 array, unrounded.
    """
    od = out_dtype or in_dtype
    A = _raw(A, "A", in_dtype); B = _raw(B, "B", in_dtype)
    bias = _raw(bias, "bias", od); R = _raw(R, "R", od); scale = _raw(scale, "scale", od)
    m_lo, m_hi = m_range if m_range is not None else (0, M)
    n_lo, n_hi = n_range if n_range is not None else (0, N)
    out = np.empty((m_hi - m_lo, n_hi - n_lo), dtype=np.float64)
    rc = lib().orc_gemm_block(M, N, K, _ptr(A), lda, int(opA), _ptr(B), ldb,
                              int(opB), in_dtype, _ptr(scale), _ptr(bias),
                              int(bool(relu)), _ptr(R), ldr, od,
                              m_lo, m_hi, n_lo, n_hi, _ptr(out),
                              threads or default_threads())
    if rc != 0:
        raise ValueError("oracle gemm_block: bad arguments")
    return out


def gemm_cells(M, N, K, A, lda, opA, B, ldb, opB, in_dtype, ms, ns, bias=None,
               relu=False, R=None, ldr=0, out_dtype=None, scale=None,
               threads=None) -> np.ndarray:
    """fp64 reference of the scattered cells (ms[i], ns[i]), one by one."""
    od = out_dtype or in_dtype
    A = _raw(A, "A", in_dtype); B = _raw(B, "B", in_dtype)
    bias = _raw(bias, "bias", od); R = _raw(R, "R", od); scale = _raw(scale, "scale", od)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    rc = lib().orc_gemm_cells(M, N, K, _ptr(A), lda, int(opA), _ptr(B), ldb,
                              int(opB), in_dtype, _ptr(scale), _ptr(bias),
                              int(bool(relu)), _ptr(R), ldr, od,
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
    refb = round_out(Cref, out_dtype)
    den = np.linalg.norm(Cref)
    return {
        "ok": ok,
        "n": int(C.size),
        "violations": int((~finite).sum() + (finite & (err > bound)).sum()),
        "max_abs": float(np.nanmax(err)) if C.size else 0.0,
        "max_rel": float(np.nanmax(err / np.maximum(np.abs(Cref), 1e-30))) if C.size else 0.0,
        "frob_rel": float(np.linalg.norm(np.nan_to_num(C - Cref)) / den) if den > 0 else 0.0,
        "bit_match": float((np.asarray(C_bits, dtype=_bits_type(out_dtype)) == refb).mean())
        if C.size else 1.0,
    }
