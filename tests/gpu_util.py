"""Test helpers: move seeded host buffers to the GPU, call the library through
its C ABI, read results back with guard bands, and judge them with the oracle.
"""
import numpy as np
import torch

import oracle
import thread_register_tile_amd as trt
import workloads as W

GUARD = 2048            # elements of sentinel before and after C
# finite patterns the kernel never writes by chance: 16-bit and binary32 outputs
SENTINEL = {W.F16: 0x7BAD, W.BF16: 0x7BAD, W.F32: 0x7BAD7BAD}


def to_dev(bits):
    if bits is None:
        return None
    if bits.dtype == np.uint32:
        return torch.from_numpy(bits.view(np.int32)).to("cuda")
    return torch.from_numpy(bits.view(np.int16)).to("cuda")


class Run:
    """One GEMM call on device copies of a workload's host buffers."""

    def __init__(self, w: W.Workload, inputs=None, ldc=None):
        self.w = w
        self.host = inputs if inputs is not None else W.make_inputs(w)
        self.A = to_dev(self.host["A"])
        self.B = to_dev(self.host["B"])
        self.bias = to_dev(self.host["bias"])
        self.R = to_dev(self.host["R"])
        self.scale = to_dev(self.host.get("scale"))
        self.ldc = ldc or w.ldc_
        n_c = (w.M - 1) * self.ldc + w.N
        self.sentinel = SENTINEL[w.odt]
        self.esize = W.ELEM_BYTES[w.odt]
        tdt = torch.int32 if self.esize == 4 else torch.int16
        self.Cbuf = torch.full((n_c + 2 * GUARD,), self.sentinel - (1 << 32 if self.esize == 4 and
                                                                  self.sentinel >= 1 << 31 else 0),
                               dtype=tdt, device="cuda")

    def c_ptr(self):
        return self.Cbuf.data_ptr() + self.esize * GUARD

    def launch(self, tile=None):
        w = self.w
        if w.regtile is not None:
            lm, ln, mt = w.regtile
            trt.gemm_regtile_raw(
                w.M, w.N, w.K, self.A.data_ptr(), w.lda_, w.opA, self.B.data_ptr(), w.ldb_,
                w.opB, self.c_ptr(), self.ldc, w.dtype, w.odt, lm, ln, mt,
                bias=self.bias.data_ptr() if self.bias is not None else 0, relu=w.relu,
                residual=self.R.data_ptr() if self.R is not None else 0,
                ldr=w.ldr_ if self.R is not None else 0,
                scale=self.scale.data_ptr() if self.scale is not None else 0,
                stream=torch.cuda.current_stream().cuda_stream)
            return
        trt.gemm_raw(w.M, w.N, w.K, self.A.data_ptr(), w.lda_, w.opA, self.B.data_ptr(),
                     w.ldb_, w.opB, self.c_ptr(), self.ldc, w.dtype, w.odt,
                     bias=self.bias.data_ptr() if self.bias is not None else 0,
                     relu=w.relu,
                     residual=self.R.data_ptr() if self.R is not None else 0,
                     ldr=w.ldr_ if self.R is not None else 0,
                     scale=self.scale.data_ptr() if self.scale is not None else 0,
                     tile=tile if tile is not None else w.tile,
                     stream=torch.cuda.current_stream().cuda_stream)

    def launch_ws(self, workspace, workspace_bytes):
        """trt_gemm_ws on the same buffers; workspace: a device address (int)."""
        w = self.w
        trt.gemm_ws_raw(w.M, w.N, w.K, self.A.data_ptr(), w.lda_, w.opA, self.B.data_ptr(),
                        w.ldb_, w.opB, self.c_ptr(), self.ldc, w.dtype, w.odt,
                        bias=self.bias.data_ptr() if self.bias is not None else 0, relu=w.relu,
                        residual=self.R.data_ptr() if self.R is not None else 0,
                        ldr=w.ldr_ if self.R is not None else 0,
                        scale=self.scale.data_ptr() if self.scale is not None else 0,
                        workspace=workspace, workspace_bytes=workspace_bytes,
                        stream=torch.cuda.current_stream().cuda_stream)

    def launch_noalloc(self):
        """trt_gemm_noalloc on the same buffers (its workspace is the library's own)."""
        w = self.w
        trt.gemm_noalloc_raw(w.M, w.N, w.K, self.A.data_ptr(), w.lda_, w.opA, self.B.data_ptr(),
                             w.ldb_, w.opB, self.c_ptr(), self.ldc, w.dtype, w.odt,
                             bias=self.bias.data_ptr() if self.bias is not None else 0,
                             relu=w.relu,
                             residual=self.R.data_ptr() if self.R is not None else 0,
                             ldr=w.ldr_ if self.R is not None else 0,
                             scale=self.scale.data_ptr() if self.scale is not None else 0,
                             stream=torch.cuda.current_stream().cuda_stream)

    def result(self):
        """C as an (M, N) array of raw bits (uint16, or uint32 for binary32
        output); asserts guards and ldc padding intact."""
        torch.cuda.synchronize()
        ut = np.uint32 if self.esize == 4 else np.uint16
        buf = self.Cbuf.cpu().numpy().view(ut)
        w = self.w
        SENT = ut(self.sentinel)
        assert (buf[:GUARD] == SENT).all(), "write before C"
        assert (buf[-GUARD:] == SENT).all(), "write after C"
        body = buf[GUARD:-GUARD]
        full = np.full(w.M * self.ldc, SENT, dtype=ut)
        full[:body.size] = body
        full = full.reshape(w.M, self.ldc)
        if self.ldc > w.N:
            pad = full[:-1, w.N:] if w.M > 1 else full[:0, w.N:]
            assert (pad == SENT).all(), "write into ldc padding"
        return np.ascontiguousarray(full[:, :w.N])


def oracle_args(w: W.Workload, host):
    return dict(M=w.M, N=w.N, K=w.K, A=host["A"], lda=w.lda_, opA=w.opA, B=host["B"],
                ldb=w.ldb_, opB=w.opB, in_dtype=w.dtype, bias=host["bias"], relu=w.relu,
                R=host["R"], ldr=w.ldr_ if host["R"] is not None else 0,
                out_dtype=w.odt, scale=host.get("scale"))


def reference_block(w, host, m_range=None, n_range=None):
    return oracle.gemm_block(**oracle_args(w, host), m_range=m_range, n_range=n_range)


def reference_cells(w, host, ms, ns):
    return oracle.gemm_cells(**oracle_args(w, host), ms=ms, ns=ns)


def assert_full_output(w, host, C, n_block=None, what=""):
    """Every element of C (M x N raw bits) against the oracle, under the
    tolerance; in column blocks of n_block when given (the oracle decodes the
    B columns of a block once, so a block bounds its memory)."""
    n_block = n_block or w.N
    for n0 in range(0, w.N, n_block):
        nr = (n0, min(w.N, n0 + n_block))
        ref = reference_block(w, host, None, nr)
        assert_accept(np.ascontiguousarray(C[:, nr[0]:nr[1]]), ref, w.odt,
                      what=f"{what or w.name} columns {nr}")
        del ref


def assert_accept(C_bits, Cref, dtype, exact=False, what=""):
    rep = oracle.accept(C_bits, Cref, dtype)
    assert rep["ok"], f"{what}: {rep}"
    if exact:
        assert rep["bit_match"] == 1.0, f"{what}: exact mode not bit-exact: {rep}"
    return rep


def sample_cells(w, n_random, seed=0):
    """Random cells plus every corner and the last row / column of the domain."""
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, w.M, n_random))
    ns = list(rng.integers(0, w.N, n_random))
    for m in (0, w.M - 1):
        for n in (0, w.N - 1):
            ms.append(m); ns.append(n)
    for i in range(min(w.N, 64)):
        ms.append(w.M - 1); ns.append(w.N - 1 - i)
    for i in range(min(w.M, 64)):
        ms.append(w.M - 1 - i); ns.append(w.N - 1)
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
