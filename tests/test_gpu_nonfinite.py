"""Non-finite values stay where the ownership maps put them.

A NaN planted at A[m, k] must turn exactly row m of C into NaN, and an Inf
at B[k, n] exactly column n into Inf or NaN; every other element must be
bit-identical to the result without them.  A wrong fragment, swizzle or
ownership map anywhere would carry the non-finite value into other rows or
columns.  Checked on every kernel family through the C ABI.
"""
import pytest
import torch

import thread_register_tile_amd as trt

pytestmark = pytest.mark.gpu

CASES = [  # (M, N, K, dtype, call)
    (600, 520, 200, torch.float16, dict(tile=(256, 256, 32))),       # pipelined, 8 waves
    (600, 520, 200, torch.bfloat16, dict(tile=(256, 192, 32))),      # pipelined, 256x192
    (300, 260, 100, torch.bfloat16, dict(tile=(64, 64, 64))),         # generic kernel
    (100, 90, 70, torch.float16, dict(tile=(16, 64, 32))),            # one-wave tile
    (12, 4096, 512, torch.float16, dict()),                           # M <= 16 streaming kernel
    (300, 200, 100, torch.float32, dict()),                           # binary32, direct copies
    (301, 203, 101, torch.float32, dict()),                           # binary32, register-staged
    (97, 83, 61, torch.float16, dict(regtile=(3, 17, 32))),           # vector lanes
    (130, 70, 40, torch.float32, dict(regtile=(64, 64, 64))),         # vector lanes, prefetched
]


def run(A, B, call):
    if "regtile" in call:
        lm, ln, mt = call["regtile"]
        return trt.gemm_regtile(A, B, lm=lm, ln=ln, max_threads=mt)
    return trt.gemm(A, B, **call)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_nonfinite_values_stay_in_their_row_and_column(case):
    M, N, K, dt, call = CASES[case]
    g = torch.Generator().manual_seed(100 + case)
    A = (torch.rand(M, K, generator=g) - 0.5).to(dt).cuda()
    B = (torch.rand(K, N, generator=g) - 0.5).to(dt).cuda()
    ref = run(A, B, call)
    m, k, n, k2 = M // 3, K // 2, (2 * N) // 3, K - 1
    A2, B2 = A.clone(), B.clone()
    A2[m, k] = float("nan")
    B2[k2, n] = float("inf")
    out = run(A2, B2, call)
    torch.cuda.synchronize()
    ref, out = ref.float().cpu(), out.float().cpu()
    assert torch.isnan(out[m]).all(), "row of the NaN"
    col = torch.cat([out[:m, n], out[m + 1:, n]])
    assert (~torch.isfinite(col)).all(), "column of the Inf"
    keep = torch.ones(M, N, dtype=torch.bool)
    keep[m, :] = False
    keep[:, n] = False
    assert torch.isfinite(out[keep]).all(), "non-finite value outside its row and column"
    assert torch.equal(out[keep], ref[keep]), "other elements changed"
