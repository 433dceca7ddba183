"""GPU parity of the split-K streaming path (trt_gemm_ws), through the C ABI.

For M <= 16 with a workspace, K is cut into slices over workgroups, fp32
partial sums of each slice go to the workspace and a second kernel adds them
in slice order and applies the epilogue.  Exact mode (operands in {-1, 0, 1},
epilogue terms in {-2..2}) makes every partial and total sum exact, so the
result must equal the oracle rounded once, bit for bit, whatever the slices;
the full skinny workload is compared element by element under the tolerance.
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


def workspace_for(w, extra=0):
    n = trt.workspace_size(w.M, w.N, w.K, w.opA, w.opB, w.dtype)
    buf = torch.full((max(n + extra, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    return n, buf


def test_split_shapes_exact():
    # every M up to 16, panels past N, slices of unequal length, epilogue
    # combinations, both input dtypes, all output dtypes, padded ldc
    rng = np.random.default_rng(31)
    for trial in range(36):
        M = 1 + trial % 16
        N = 4 * int(rng.integers(1, 700))
        K = 8 * int(rng.integers(64, 900))     # at least 16 iterations of 32: two slices
        dt = W.F16 if trial % 3 else W.BF16
        odt = [dt, W.F32, W.BF16 if dt == W.F16 else W.F16][trial % 3]
        w = W.Workload("split", M, N, K, lda=K + 8 * (trial % 2), ldb=N + 4 * (trial % 3),
                       dtype=dt, out_dtype=odt, dist="ternary", seed=7000 + trial,
                       bias=bool(trial % 2), relu=bool(trial % 4 == 1),
                       residual=bool(trial % 3 == 0), row_scale=bool(trial % 5 == 2))
        need, ws = workspace_for(w)
        assert need > 0, (M, N, K)
        run = Run(w, ldc=N + (trial % 5))
        run.launch_ws(ws.data_ptr(), ws.numel() * 4)
        assert_accept(run.result(), reference_block(w, run.host), odt, exact=True,
                      what=f"M={M} N={N} K={K} dt={dt} odt={odt}")


def test_skinny_workload_split_full_size():
    # the whole output, element by element, in column blocks of 4096
    w = W.SKINNY
    need, ws = workspace_for(w)
    assert need == 8 * 16 * 16384 * 4
    run = Run(w)
    run.launch_ws(ws.data_ptr(), need)
    assert_full_output(w, run.host, run.result(), n_block=4096, what="skinny, split K")


def test_split_is_deterministic_and_matches_unsplit_exactly():
    # two split runs are bit-identical; in exact mode they also equal the
    # single-pass kernel's result bit for bit
    w = replace(W.SKINNY, N=4096, dist="ternary", seed=91, bias=True, relu=True)
    need, ws = workspace_for(w)
    run = Run(w)
    run.launch_ws(ws.data_ptr(), need)
    c1 = run.result()
    run.launch_ws(ws.data_ptr(), need)
    c2 = run.result()
    run.launch()
    c3 = run.result()
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)


def test_ws_call_without_split_leaves_workspace_alone():
    # shapes that do not split run trt_gemm's kernels; the workspace may be
    # absent and is not written when given
    for w in (replace(W.SQUARE, M=256, N=256, K=128, dist="ternary"),
              W.Workload("short-k", 16, 512, 64, dist="ternary", seed=3)):
        assert trt.workspace_size(w.M, w.N, w.K, w.opA, w.opB, w.dtype) == 0
        run = Run(w)
        run.launch_ws(0, 0)
        assert_accept(run.result(), reference_block(w, run.host), w.odt, exact=True)
        sentinel = torch.full((1024,), 7.0, device="cuda")
        run.launch_ws(sentinel.data_ptr(), 4096)
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all())
