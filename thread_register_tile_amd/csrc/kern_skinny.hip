// kern_skinny.hip -- instances of the streaming kernel for M <= 16.
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

}  // namespace trt
