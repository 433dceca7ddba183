// kern_dma256_f16_am.hip -- instances of the pipelined direct-to-LDS
// kernel (256x256 tile of 8 waves, K step 32, 16x16x32 fragments) for f16 inputs with
// A stored transposed (m contiguous), in a translation unit of their own so that the
// library builds in parallel.
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

template void launch_pipelined_a<Tile256D, DT_F16, false>(GemmArgs, bool, hipStream_t);

}  // namespace trt
