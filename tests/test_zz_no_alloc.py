"""GPU test of trt_gemm_noalloc, the allocation-free variant of trt_gemm_ws.

Through the C ABI: on the same inputs it must give trt_gemm_ws's result bit
for bit (same kernels, same split plan, its workspace the library's own
scratch array instead of the caller's), and the oracle's result (exact mode,
so bit for bit).  Two calls in a row, the second on a smaller problem, so that
the scratch array still holds the first call's partial sums when the second
one runs; and a shape that needs no workspace.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import thread_register_tile_amd as trt
import workloads as W

from gpu_util import Run, assert_accept, assert_full_output, reference_block

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    trt.lib()


def _against_workspace_entry(w, n_block=None):
    need = trt.workspace_size(w.M, w.N, w.K, w.opA, w.opB, w.dtype)
    print(f"noalloc: {w.name} {w.M}x{w.N}x{w.K}, workspace {need} bytes", flush=True)
    run = Run(w)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    run.launch_ws(ws.data_ptr(), need)
    with_ws = run.result()
    run2 = Run(w, inputs=run.host)
    run2.launch_noalloc()
    got = run2.result()
    assert np.array_equal(got, with_ws), f"{w.name}: noalloc differs from trt_gemm_ws"
    assert_full_output(w, run2.host, got, n_block=n_block, what=f"{w.name} noalloc")
    return need


def test_noalloc_two_calls_then_smaller():
    big = replace(W.SKINNY, dist="ternary", seed=95, bias=True, relu=True)
    small = W.Workload("noalloc-small", 7, 2048, 4096, dtype=W.BF16, out_dtype=W.F32,
                       bias=True, residual=True, row_scale=True, dist="ternary", seed=96)
    assert _against_workspace_entry(big, n_block=4096) == 8 * 16 * 16384 * 4
    n_small = _against_workspace_entry(small)
    assert 0 < n_small < 8 * 16 * 16384 * 4


def test_noalloc_without_split():
    # a shape that needs no workspace runs trt_gemm's kernels
    w = W.Workload("noalloc-square", 300, 260, 200, dist="ternary", seed=97, bias=True)
    assert trt.workspace_size(w.M, w.N, w.K) == 0
    run = Run(w)
    run.launch_noalloc()
    assert_accept(run.result(), reference_block(w, run.host), w.odt, exact=True)
