"""The entry points under HIP graph capture.

The library enqueues kernels only (no allocation, no memset, no host
synchronisation), so its calls can be captured into a graph and replayed.
Each replay, with eager work and synchronisations between replays, must
reproduce the eager results bit for bit (every kernel here is deterministic).
"""
import numpy as np
import pytest
import torch

import thread_register_tile_amd as trt
import workloads as W

pytestmark = pytest.mark.gpu


def bits_tensor(w, tensor_id, rows, cols, dtype):
    x = W._draw(w, tensor_id, rows, cols)
    b = W.to_bits(x, dtype)
    return torch.from_numpy(b.view(np.int32 if b.dtype == np.uint32 else np.int16)).cuda()


def make_calls():
    """A list of (launch(stream), output tensor) covering every kernel family."""
    calls = []
    specs = [  # (M, N, K, dtype, tile, epilogue)
        (64, 64, 32, W.F16, (16, 64, 32), False),       # generic 16x64 tile
        (1024, 768, 512, W.BF16, None, True),           # pipelined 256-wide tiles
        (16, 4096, 2048, W.F16, None, False),           # M <= 16 streaming kernel
        (300, 200, 100, W.F32, None, True),             # binary32 operands
    ]
    for i, (M, N, K, dt, tile, epi) in enumerate(specs):
        w = W.Workload("graph", M, N, K, dtype=dt, dist="uniform", seed=50 + i)
        A = bits_tensor(w, 0, M, K, dt)
        B = bits_tensor(w, 1, K, N, dt)
        bias = bits_tensor(w, 2, 1, N, dt) if epi else None
        R = bits_tensor(w, 3, M, N, dt) if epi else None
        C = torch.empty(M * N, dtype=A.dtype, device="cuda")

        def launch(s, M=M, N=N, K=K, A=A, B=B, C=C, dt=dt, bias=bias, R=R, tile=tile):
            trt.gemm_raw(M, N, K, A.data_ptr(), K, 0, B.data_ptr(), N, 0, C.data_ptr(), N, dt, dt,
                         bias=bias.data_ptr() if bias is not None else 0, relu=bias is not None,
                         residual=R.data_ptr() if R is not None else 0,
                         ldr=N if R is not None else 0, tile=tile, stream=s)
        calls.append((launch, C))
    # the register-tile GEMM on vector lanes
    w = W.Workload("graph-rt", 97, 83, 61, dtype=W.F16, dist="uniform", seed=60)
    A = bits_tensor(w, 0, 97, 61, W.F16)
    B = bits_tensor(w, 1, 61, 83, W.F16)
    C = torch.empty(97 * 83, dtype=torch.int16, device="cuda")
    calls.append((lambda s: trt.gemm_regtile_raw(97, 83, 61, A.data_ptr(), 61, 0, B.data_ptr(),
                                                 83, 0, C.data_ptr(), 83, W.F16, W.F16, 3, 17,
                                                 32, stream=s), C))
    # the block reduction
    x = bits_tensor(W.Workload("graph-red", 1, 1, 1, dist="normal", seed=61), 0, 1, 100003,
                    W.F16)
    out = torch.empty(-(-100003 // 1000), dtype=torch.float32, device="cuda")
    calls.append((lambda s: trt.block_reduce_raw(x.data_ptr(), 100003, 1000, W.F16,
                                                 trt.REDUCE_SUM, out.data_ptr(), stream=s), out))
    return calls


def test_capture_and_replay_matches_eager():
    calls = make_calls()
    s = torch.cuda.current_stream().cuda_stream
    for launch, _ in calls:
        launch(s)
    torch.cuda.synchronize()
    eager = [out.clone() for _, out in calls]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, out in calls:
            out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for launch, _ in calls:
                launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: clobber every output first
        for _, out in calls:
            out.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((_, out), ref) in enumerate(zip(calls, eager)):
            assert torch.equal(out, ref), f"replay {rep}, call {i} differs from the eager result"
