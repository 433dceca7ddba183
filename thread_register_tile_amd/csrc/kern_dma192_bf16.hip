// kern_dma192_bf16.hip -- instances of the pipelined direct-to-LDS kernel on
// the 256x192 tile (8x6 fragments of 16x16 per wave: a register tile that is
// not a power of two) for bf16 inputs, in a translation unit of their own.
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

template void launch_pipelined_a<Tile256x192D, DT_BF16, true>(GemmArgs, bool, hipStream_t);
template void launch_pipelined_a<Tile256x192D, DT_BF16, false>(GemmArgs, bool, hipStream_t);

}  // namespace trt
