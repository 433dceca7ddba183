"""Python binding of libtrt.so, the MI355X register-tile GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libtrt.so.  PyTorch provides device memory and the current
stream; nothing here computes on tensors.  If the library is not built, every
call raises -- there is no fallback path.

    import thread_register_tile_amd as trt
    C = trt.gemm(A, B)                          # C = A @ B
    C = trt.gemm(A, B, bias=b, relu=True, residual=R)
    C = trt.gemm(At, B, opA="T")                # A stored transposed
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtrt.so")

# status codes (include/trt.h)
OK, ERR_SIZE, ERR_STRIDE, ERR_NULL, ERR_ALIGN, ERR_OVERLAP, ERR_DTYPE, \
    ERR_UNSUPPORTED, ERR_HIP, ERR_ARG = range(10)
STATUS_NAMES = {OK: "TRT_OK", ERR_SIZE: "TRT_ERR_SIZE", ERR_STRIDE: "TRT_ERR_STRIDE",
                ERR_NULL: "TRT_ERR_NULL", ERR_ALIGN: "TRT_ERR_ALIGN",
                ERR_OVERLAP: "TRT_ERR_OVERLAP", ERR_DTYPE: "TRT_ERR_DTYPE",
                ERR_UNSUPPORTED: "TRT_ERR_UNSUPPORTED", ERR_HIP: "TRT_ERR_HIP",
                ERR_ARG: "TRT_ERR_ARG"}

F16, BF16, F32 = 1, 2, 3
OP_N, OP_T = 0, 1

MAP_C_OWNER = 0
MAP_LDS_SLOT_A = 1
MAP_LDS_SLOT_B = 2
MAP_COPY_KCONTIG_A = 3
MAP_COPY_MNCONTIG_A = 4
MAP_COPY_KCONTIG_B = 5
MAP_COPY_MNCONTIG_B = 6
MAP_DMA_KC_SLOT_A = 7
MAP_DMA_KC_SLOT_B = 8
MAP_DMA_MN_SLOT_A = 9
MAP_DMA_MN_SLOT_B = 10


class TrtError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class Epilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("relu", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("ldr", ctypes.c_int64),
                ("row_scale", ctypes.c_void_p)]


class TileDesc(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libtrt.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m thread_register_tile_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        gemm_args = [i64, i64, i64, vp, i64, i32, vp, i64, i32, vp, i64, i32, i32,
                     ctypes.POINTER(Epilogue)]
        L.trt_gemm.argtypes = gemm_args + [vp]
        L.trt_gemm.restype = i32
        L.trt_gemm_tiled.argtypes = gemm_args + [ctypes.POINTER(TileDesc), vp]
        L.trt_gemm_tiled.restype = i32
        L.trt_validate.argtypes = gemm_args + [ctypes.POINTER(TileDesc)]
        L.trt_validate.restype = i32
        L.trt_gemm_ws.argtypes = gemm_args + [vp, i64, vp]
        L.trt_gemm_ws.restype = i32
        L.trt_gemm_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
        L.trt_gemm_workspace_size.restype = i64
        L.trt_gemm_noalloc.argtypes = gemm_args + [vp]
        L.trt_gemm_noalloc.restype = i32
        L.trt_tile_count.argtypes = []
        L.trt_tile_count.restype = i32
        L.trt_tile_at.argtypes = [i32, ctypes.POINTER(TileDesc), ctypes.POINTER(i32),
                                  ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.trt_tile_at.restype = i32
        L.trt_layout_dump.argtypes = [i32, ctypes.POINTER(TileDesc), vp, vp, i64, vp]
        L.trt_layout_dump.restype = i32
        L.trt_layout_dump_host.argtypes = [i32, ctypes.POINTER(TileDesc), vp, vp, i64]
        L.trt_layout_dump_host.restype = i32
        L.trt_layout_size.argtypes = [i32, ctypes.POINTER(TileDesc)]
        L.trt_layout_size.restype = i64
        L.trt_layout_rank.argtypes = [ctypes.POINTER(TileDesc), ctypes.POINTER(i32),
                                      ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.trt_layout_rank.restype = i32
        L.trt_mfma_probe.argtypes = [i32, i32, vp, vp, vp, vp]
        L.trt_mfma_probe.restype = i32
        L.trt_hbm_read_probe.argtypes = [vp, i64, vp, i64, vp]
        L.trt_hbm_read_probe.restype = i32
        L.trt_mfma_loop_probe.argtypes = [i32, vp, i32, vp, i64, vp]
        L.trt_mfma_loop_probe.restype = i32
        L.trt_clock_probe.argtypes = [i64, vp, i64, vp]
        L.trt_clock_probe.restype = i32
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.trt_gf2_rank.argtypes = [i32, i32, u32p]
        L.trt_gf2_rank.restype = i32
        L.trt_gf2_compose.argtypes = [i32, i32, u32p, i32, i32, u32p, u32p]
        L.trt_gf2_compose.restype = i32
        L.trt_gf2_product.argtypes = [i32, i32, u32p, i32, i32, u32p, u32p]
        L.trt_gf2_product.restype = i32
        L.trt_gf2_sublayout.argtypes = [i32, i32, u32p, ctypes.c_uint32, ctypes.c_uint32, u32p,
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.trt_gf2_sublayout.restype = i32
        L.trt_gf2_invert_and_compose.argtypes = [i32, i32, u32p, i32, u32p, u32p]
        L.trt_gf2_invert_and_compose.restype = i32
        L.trt_block_reduce.argtypes = [vp, i64, i64, i32, i32, vp, vp]
        L.trt_block_reduce.restype = i32
        i32p = ctypes.POINTER(i32)
        L.trt_regtile_thread_shape.argtypes = [i32, i32, i32, i32p, i32p]
        L.trt_regtile_thread_shape.restype = i32
        L.trt_regtile_owner.argtypes = [i32, i32, i32, i32, vp, vp, i64]
        L.trt_regtile_owner.restype = i32
        L.trt_gemm_regtile.argtypes = gemm_args + [i32, i32, i32, vp]
        L.trt_gemm_regtile.restype = i32
        L.trt_choose_tile.argtypes = [i64, i64, i32, ctypes.POINTER(TileDesc)]
        L.trt_choose_tile.restype = i32
        L.trt_abi_version.argtypes = []
        L.trt_abi_version.restype = i32
        L.trt_last_error.argtypes = []
        L.trt_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().trt_last_error().decode()


def abi_version() -> int:
    return lib().trt_abi_version()


def _check(status):
    if status != OK:
        raise TrtError(status, last_error())


def _tile(tile):
    if tile is None:
        return None
    return ctypes.byref(TileDesc(*tile))


def _epi(bias_ptr, relu, res_ptr, ldr, scale_ptr=0):
    if not bias_ptr and not relu and not res_ptr and not scale_ptr:
        return None
    return ctypes.byref(Epilogue(bias_ptr or None, int(bool(relu)), res_ptr or None, ldr,
                                 scale_ptr or None))


# ---- raw entry points (pointers and sizes, as in include/trt.h) --------------

def gemm_raw(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype,
             bias=0, relu=False, residual=0, ldr=0, scale=0, tile=None, stream=0):
    """trt_gemm_tiled on raw device addresses (ints).  Raises TrtError."""
    _check(lib().trt_gemm_tiled(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                                out_dtype, _epi(bias, relu, residual, ldr, scale),
                                _tile(tile), stream or None))


def gemm_ws_raw(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype,
                bias=0, relu=False, residual=0, ldr=0, scale=0, workspace=0, workspace_bytes=0,
                stream=0):
    """trt_gemm_ws on raw device addresses (ints).  Raises TrtError."""
    _check(lib().trt_gemm_ws(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype,
                             _epi(bias, relu, residual, ldr, scale), workspace or None,
                             workspace_bytes, stream or None))


NOALLOC_SCRATCH_BYTES = 16777216   # TRT_NOALLOC_SCRATCH_BYTES


def gemm_noalloc_raw(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype,
                     bias=0, relu=False, residual=0, ldr=0, scale=0, stream=0):
    """trt_gemm_noalloc on raw device addresses (ints).  Raises TrtError."""
    _check(lib().trt_gemm_noalloc(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                                  out_dtype, _epi(bias, relu, residual, ldr, scale),
                                  stream or None))


def workspace_size(M, N, K, opA=OP_N, opB=OP_N, in_dtype=F16) -> int:
    """trt_gemm_workspace_size: bytes of workspace trt_gemm_ws uses (0: none)."""
    n = lib().trt_gemm_workspace_size(M, N, K, opA, opB, in_dtype)
    if n < 0:
        raise TrtError(ERR_ARG, last_error())
    return n


def validate_raw(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype,
                 bias=0, relu=False, residual=0, ldr=0, scale=0, tile=None) -> int:
    """trt_validate: the status a call would return, without any GPU work."""
    return lib().trt_validate(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                              out_dtype, _epi(bias, relu, residual, ldr, scale), _tile(tile))


def choose_tile(M, N, in_dtype=F16):
    """trt_choose_tile: the (BM, BN, BK) tile trt_gemm uses for an M x N output."""
    t = TileDesc()
    _check(lib().trt_choose_tile(M, N, in_dtype, ctypes.byref(t)))
    return (t.bm, t.bn, t.bk)


def tiles():
    """Compiled tiles: [(bm, bn, bk, waves_m, waves_n, regs_per_lane, frag), ...]
    where frag is the edge (16 or 32) of the matrix-core fragments."""
    out = []
    for i in range(lib().trt_tile_count()):
        t = TileDesc()
        wm, wn, regs, fr = (ctypes.c_int32() for _ in range(4))
        _check(lib().trt_tile_at(i, ctypes.byref(t), ctypes.byref(wm), ctypes.byref(wn),
                                 ctypes.byref(regs), ctypes.byref(fr)))
        out.append((t.bm, t.bn, t.bk, wm.value, wn.value, regs.value, fr.value))
    return out


def layout_size(map_id, tile) -> int:
    return lib().trt_layout_size(map_id, _tile(tile))


def layout_rank(tile):
    r, i, o = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().trt_layout_rank(_tile(tile), ctypes.byref(r), ctypes.byref(i), ctypes.byref(o)))
    return r.value, i.value, o.value


def layout_dump_host(map_id, tile):
    """Evaluate a layout map on the host: returns (rows, cols) numpy int32."""
    import numpy as np
    n = layout_size(map_id, tile)
    if n < 0:
        raise TrtError(ERR_ARG, "unknown map or tile")
    rows = np.empty(n, dtype=np.int32)
    cols = np.empty(n, dtype=np.int32)
    _check(lib().trt_layout_dump_host(map_id, _tile(tile), rows.ctypes.data,
                                      cols.ctypes.data, n))
    return rows, cols


# ---- torch-facing helpers (device memory and the current stream) ----------------

def _torch():
    import torch
    return torch


_DT = {}


def _dtype_code(t):
    torch = _torch()
    if not _DT:
        _DT.update({torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32})
    if t.dtype not in _DT:
        raise TrtError(ERR_DTYPE, f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ld(t, name):
    """Leading dimension of a 2-D tensor whose inner stride is 1."""
    if t.dim() != 2:
        raise TrtError(ERR_ARG, f"{name} must be 2-D")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise TrtError(ERR_STRIDE, f"{name} must have unit inner stride")
    return max(t.stride(0), 1)


def _gemm_call(A, B, opA, opB, bias, relu, residual, row_scale, out, out_dtype, M, N, K):
    """Shapes, dtypes and raw pointers of a GEMM on torch tensors; allocates
    `out` if it is not given.  Returns (out, positional args, keyword args)
    for gemm_raw / gemm_regtile_raw."""
    torch = _torch()
    opa = OP_T if opA in ("T", OP_T, True) else OP_N
    opb = OP_T if opB in ("T", OP_T, True) else OP_N
    M_ = A.size(1) if opa else A.size(0)
    K_ = A.size(0) if opa else A.size(1)
    N_ = B.size(0) if opb else B.size(1)
    KB = B.size(1) if opb else B.size(0)
    if KB != K_:
        raise TrtError(ERR_SIZE, f"inner dimensions differ: {K_} vs {KB}")
    M, N, K = M or M_, N or N_, K or K_
    dt = _dtype_code(A)
    if _dtype_code(B) != dt:
        raise TrtError(ERR_DTYPE, "A and B dtypes differ")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or A.dtype, device=A.device)
    odt = _dtype_code(out)
    for name, t, need in (("bias", bias, N), ("row_scale", row_scale, M)):
        if t is None:
            continue
        if t.dtype != out.dtype:
            raise TrtError(ERR_DTYPE, f"{name} must have the output dtype {out.dtype}")
        if not t.is_contiguous() or t.numel() < need:
            raise TrtError(ERR_SIZE, f"{name} must be contiguous with at least {need} elements")
    ldr = 0
    if residual is not None:
        if residual.dtype != out.dtype:
            raise TrtError(ERR_DTYPE, f"residual must have the output dtype {out.dtype}")
        if residual.dim() != 2 or residual.size(0) < M or residual.size(1) < N:
            raise TrtError(ERR_SIZE, f"residual must be at least [{M}, {N}]")
        ldr = _ld(residual, "residual")
    args = (M, N, K, A.data_ptr(), _ld(A, "A"), opa, B.data_ptr(), _ld(B, "B"), opb,
            out.data_ptr(), _ld(out, "out"), dt, odt)
    kw = dict(bias=bias.data_ptr() if bias is not None else 0, relu=relu,
              residual=residual.data_ptr() if residual is not None else 0, ldr=ldr,
              scale=row_scale.data_ptr() if row_scale is not None else 0,
              stream=_stream(A.device))
    return out, args, kw


def gemm(A, B, *, opA="N", opB="N", bias=None, relu=False, residual=None, row_scale=None,
         out=None, out_dtype=None, tile=None, M=None, N=None, K=None):
    """C = relu((A.B) * row_scale[:, None] + bias) + residual on the GPU, in one kernel.

    A is [M, K] (opA="N") or its transpose stored as [K, M] (opA="T"); B is
    [K, N] (opB="N") or stored as [N, K] (opB="T"); A and B share one dtype,
    float16, bfloat16 or float32.  Tensors may be
    row-padded views (unit inner stride, any row stride).  bias is [N],
    row_scale [M], residual [M, N], all of the output dtype: out's dtype if
    out is given, else out_dtype (a torch dtype: float16, bfloat16 or
    float32), else A's dtype.  out, if given, is written; otherwise a new
    [M, N] tensor is returned.  Runs on torch's current stream; no
    synchronisation.
    """
    out, args, kw = _gemm_call(A, B, opA, opB, bias, relu, residual, row_scale, out, out_dtype,
                               M, N, K)
    gemm_raw(*args, tile=tile, **kw)
    return out


def gemm_regtile(A, B, *, lm, ln, max_threads=None, opA="N", opB="N", bias=None, relu=False,
                 residual=None, row_scale=None, out=None, out_dtype=None):
    """gemm() computed on vector lanes with a register tile of logical shape
    (lm, ln) and the thread shape regtile_thread_shape(lm, ln, max_threads)
    (trt_gemm_regtile).  Same arguments and result as gemm()."""
    out, args, kw = _gemm_call(A, B, opA, opB, bias, relu, residual, row_scale, out, out_dtype,
                               None, None, None)
    gemm_regtile_raw(*args, lm, ln, max_threads or REGTILE_MAX_THREADS, **kw)
    return out


def layout_dump(map_id, tile, device="cuda"):
    """Evaluate a layout map with the kernels' device functions; returns
    (rows, cols) as int32 tensors on `device`."""
    torch = _torch()
    n = layout_size(map_id, tile)
    if n < 0:
        raise TrtError(ERR_ARG, "unknown map or tile")
    rows = torch.empty(n, dtype=torch.int32, device=device)
    cols = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().trt_layout_dump(map_id, _tile(tile), rows.data_ptr(), cols.data_ptr(), n,
                                 _stream(rows.device)))
    return rows, cols


def mfma_probe(a_regs, b_regs, dtype=F16, shape=16):
    """Run one matrix-core instruction (shape 16: 16x16x32, 32: 32x32x16):
    a_regs, b_regs are [64, 8] 16-bit tensors (lane-major operand registers);
    returns [64, 4] (shape 16) or [64, 16] (shape 32) fp32."""
    torch = _torch()
    c = torch.empty((64, 4 if shape == 16 else 16), dtype=torch.float32, device=a_regs.device)
    a = a_regs.contiguous()
    b = b_regs.contiguous()
    _check(lib().trt_mfma_probe(dtype, shape, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                _stream(a.device)))
    return c


READ_PROBE_SINK_BYTES = 32768   # TRT_READ_PROBE_SINK_BYTES


def hbm_read_probe_raw(x, nbytes, sink, sink_bytes, stream=0):
    """trt_hbm_read_probe on raw device addresses; raises TrtError on error."""
    _check(lib().trt_hbm_read_probe(x, nbytes, sink, sink_bytes, stream))


def hbm_read_probe(x, sink=None):
    """Stream-read the bytes of device tensor x once (a bandwidth yardstick);
    returns the [2048, 16]-byte digest tensor (uint8), whose XOR over rows is
    the XOR of x's 16-byte words."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(READ_PROBE_SINK_BYTES, dtype=torch.uint8, device=x.device)
    hbm_read_probe_raw(x.data_ptr(), x.numel() * x.element_size(), sink.data_ptr(),
                       sink.numel() * sink.element_size(), _stream(x.device))
    return sink.view(-1, 16)


MFMA_PROBE_OPERAND_BYTES = 16384   # TRT_MFMA_PROBE_OPERAND_BYTES
MFMA_PROBE_SINK_BYTES = 4194304    # TRT_MFMA_PROBE_SINK_BYTES


def mfma_loop_probe_raw(dtype, operands, iters, sink, sink_bytes, stream=0):
    """trt_mfma_loop_probe on raw device addresses; raises TrtError on error."""
    _check(lib().trt_mfma_loop_probe(dtype, operands, iters, sink, sink_bytes, stream))


def mfma_loop_probe(operands, iters, dtype=F16, sink=None):
    """Run the matrix-core yardstick on a device tensor of 16 KiB of operand
    data; returns the [256*256, 16] fp32 sums (one row per thread)."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(MFMA_PROBE_SINK_BYTES // 4, dtype=torch.float32,
                           device=operands.device)
    mfma_loop_probe_raw(dtype, operands.data_ptr(), iters, sink.data_ptr(),
                        sink.numel() * sink.element_size(), _stream(operands.device))
    return sink.view(-1, 16)


def mfma_loop_probe_flops(iters, dtype=F16):
    """FLOPs of one trt_mfma_loop_probe launch."""
    if dtype == F32:
        return 256 * 4 * iters * 32 * (2 * 16 * 16 * 4)
    return 256 * 4 * iters * 64 * (2 * 16 * 16 * 32)


CLOCK_PROBE_SINK_BYTES = 4096     # TRT_CLOCK_PROBE_SINK_BYTES


def clock_probe_raw(ticks, sink, sink_bytes, stream=0):
    """trt_clock_probe on a raw device address; raises TrtError on error."""
    _check(lib().trt_clock_probe(ticks, sink, sink_bytes, stream))


def clock_probe(ticks, device="cuda", sink=None):
    """Run the clock yardstick once on the current stream; returns the device
    tensor of [256, 2] int64 (shader cycles, real-time ticks) per workgroup."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(CLOCK_PROBE_SINK_BYTES // 8, dtype=torch.int64, device=device)
    clock_probe_raw(ticks, sink.data_ptr(), sink.numel() * sink.element_size(),
                    _stream(sink.device))
    return sink.view(-1, 2)


# ---- the GF(2) layout algebra (host only; maps as lists of column words) -------

def _u32(cols):
    arr = (ctypes.c_uint32 * max(len(cols), 1))(*[int(c) for c in cols])
    return arr


def gf2_rank(cols, nout):
    r = lib().trt_gf2_rank(len(cols), nout, _u32(cols))
    if r < 0:
        raise TrtError(ERR_ARG, last_error())
    return r


def gf2_compose(outer, outer_nout, inner, inner_nout):
    """outer o inner (outer has inner_nout input bits)."""
    out = (ctypes.c_uint32 * max(len(inner), 1))()
    _check(lib().trt_gf2_compose(len(outer), outer_nout, _u32(outer), len(inner), inner_nout,
                                 _u32(inner), out))
    return list(out)[:len(inner)]


def gf2_product(a, a_nout, b, b_nout):
    out = (ctypes.c_uint32 * max(len(a) + len(b), 1))()
    _check(lib().trt_gf2_product(len(a), a_nout, _u32(a), len(b), b_nout, _u32(b), out))
    return list(out)[:len(a) + len(b)]


def gf2_sublayout(cols, nout, in_mask, out_mask):
    """Returns (columns, nin, nout) of the restricted, projected map."""
    out = (ctypes.c_uint32 * 32)()
    ni, no = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().trt_gf2_sublayout(len(cols), nout, _u32(cols), in_mask, out_mask, out,
                                   ctypes.byref(ni), ctypes.byref(no)))
    return list(out)[:ni.value], ni.value, no.value


def gf2_invert_and_compose(R, S, t_bits):
    """Q with S(Q(x)) == R(x); raises TrtError (ERR_ARG) when R leaves S's image."""
    out = (ctypes.c_uint32 * max(len(R), 1))()
    _check(lib().trt_gf2_invert_and_compose(len(R), t_bits, _u32(R), len(S), _u32(S), out))
    return list(out)[:len(R)]


# ---- the rank-1 block reduction ---------------------------------------------------

# ---- register tiles of any logical shape -------------------------------------

REGTILE_MAX_THREADS = 64     # one wavefront per tile
REGTILE_MAX_REGS = 8         # registers per axis


def regtile_thread_shape(lm, ln, max_threads=REGTILE_MAX_THREADS):
    """trt_regtile_thread_shape: the physical thread shape (tm, tn) the
    deterministic policy picks for a logical (lm, ln) tile."""
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().trt_regtile_thread_shape(lm, ln, max_threads, ctypes.byref(tm),
                                          ctypes.byref(tn)))
    return tm.value, tn.value


def regtile_owner(lm, ln, tm, tn):
    """trt_regtile_owner: (rows, cols) int32 arrays indexed by
    thread * registers_per_thread + register."""
    import numpy as np
    n = lm * ln
    rows = np.empty(max(n, 1), dtype=np.int32)
    cols = np.empty(max(n, 1), dtype=np.int32)
    _check(lib().trt_regtile_owner(lm, ln, tm, tn, rows.ctypes.data, cols.ctypes.data, n))
    return rows[:n], cols[:n]


def gemm_regtile_raw(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, lm, ln,
                     max_threads=REGTILE_MAX_THREADS, bias=0, relu=False, residual=0, ldr=0,
                     scale=0, stream=0):
    """trt_gemm_regtile on raw device addresses (ints).  Raises TrtError."""
    _check(lib().trt_gemm_regtile(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                                  out_dtype, _epi(bias, relu, residual, ldr, scale), lm, ln,
                                  max_threads, stream or None))


REDUCE_SUM, REDUCE_MAX, REDUCE_MIN = 0, 1, 2


def block_reduce_raw(x, n, block, dtype, op, out, stream=0):
    """trt_block_reduce on raw device addresses; raises TrtError on error."""
    _check(lib().trt_block_reduce(x, n, block, dtype, op, out, stream or None))


def block_reduce(x, block, op=REDUCE_SUM, out=None):
    """out[b] = op over each block of `block` consecutive elements of the 1-D
    device tensor x (float16, bfloat16 or float32); returns float32 [nblocks]."""
    torch = _torch()
    n = x.numel()
    nb = -(-n // block)
    if out is None:
        out = torch.empty(nb, dtype=torch.float32, device=x.device)
    block_reduce_raw(x.data_ptr(), n, block, _dtype_code(x), op, out.data_ptr(), _stream(x.device))
    return out
