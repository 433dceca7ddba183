// kern_skinny.hip -- instances of the streaming kernels for M <= 16: the
// single-pass one, and the split-K pair that uses a workspace.
#include "gemm_skinny.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

hipError_t launch_skinny(GemmArgs a, int dt, hipStream_t s) {
  const dim3 grid((a.N + SkinnyTile::BN - 1) / SkinnyTile::BN);
  const dim3 block(SkinnyTile::THREADS);
  if (dt == DT_F16) return launch(gemm_skinny_kernel<DT_F16>, grid, block, 0, s, a);
  return launch(gemm_skinny_kernel<DT_BF16>, grid, block, 0, s, a);
}

hipError_t launch_skinny_split(GemmArgs a, int dt, float* ws, int splits, int per_split,
                               hipStream_t s) {
  const int panels = (a.N + SkinnySplit::PANEL - 1) / SkinnySplit::PANEL;
  const dim3 grid((unsigned)(panels * splits)), block(SkinnySplit::THREADS);
  const hipError_t e =
      dt == DT_F16 ? launch(gemm_skinny_split_kernel<DT_F16>, grid, block, 0, s, a, ws, splits, per_split)
                   : launch(gemm_skinny_split_kernel<DT_BF16>, grid, block, 0, s, a, ws, splits, per_split);
  if (e != hipSuccess) return e;
  const int64_t runs = (int64_t)a.M * (a.N / 4);
  const dim3 rgrid((unsigned)((runs + 255) / 256)), rblock(256);
  const float* wsc = ws;
  if (a.out_dt == DT_F16) return launch(skinny_split_reduce_kernel<DT_F16>, rgrid, rblock, 0, s, a, wsc, splits);
  if (a.out_dt == DT_BF16) return launch(skinny_split_reduce_kernel<DT_BF16>, rgrid, rblock, 0, s, a, wsc, splits);
  return launch(skinny_split_reduce_kernel<DT_F32>, rgrid, rblock, 0, s, a, wsc, splits);
}

}  // namespace trt
