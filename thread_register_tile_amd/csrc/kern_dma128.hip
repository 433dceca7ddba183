// kern_dma128.hip -- instances of the pipelined kernel on the 128x128x32 tile
// (4 waves of 4x4 fragments of 16x16, two workgroups per compute unit), for
// problems too small to give every compute unit a 256-wide tile.
#include "gemm_dma.hpp"
#include "tiles.hpp"

namespace trt {

template <class TL, int DT, bool A_KC>
void launch_pipelined_a(GemmArgs a, bool b_kc, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n);
  const dim3 block(TL::THREADS);
  if (b_kc)
    hipLaunchKernelGGL((gemm_dma_kernel<TL, DT, A_KC, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_dma_kernel<TL, DT, A_KC, false>), grid, block, 0, s, a);
}

template void launch_pipelined_a<Tile128D, DT_F16, true>(GemmArgs, bool, hipStream_t);
template void launch_pipelined_a<Tile128D, DT_F16, false>(GemmArgs, bool, hipStream_t);
template void launch_pipelined_a<Tile128D, DT_BF16, true>(GemmArgs, bool, hipStream_t);
template void launch_pipelined_a<Tile128D, DT_BF16, false>(GemmArgs, bool, hipStream_t);

}  // namespace trt
