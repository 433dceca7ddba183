// kern_dma256.hip -- instances of the pipelined direct-to-LDS kernel
// (256x256 tile, K step 32, 32x32x16 fragments), in a translation unit of
// their own so that the library builds in parallel.
#include "gemm_dma.hpp"
#include "tiles.hpp"

namespace trt {

template <class TL>
void launch_pipelined(GemmArgs a, int dt, int opA, int opB, hipStream_t s) {
  a.tiles_m = (a.M + TL::BM - 1) / TL::BM;
  a.tiles_n = (a.N + TL::BN - 1) / TL::BN;
  const dim3 grid(a.tiles_m * a.tiles_n);
  const dim3 block(TL::THREADS);
  const bool akc = opA == 0, bkc = opB == 1;
  if (dt == DT_F16) {
    if (akc && bkc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_F16, true, true>), grid, block, 0, s, a);
    else if (akc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_F16, true, false>), grid, block, 0, s, a);
    else if (bkc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_F16, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_F16, false, false>), grid, block, 0, s, a);
  } else {
    if (akc && bkc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_BF16, true, true>), grid, block, 0, s, a);
    else if (akc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_BF16, true, false>), grid, block, 0, s, a);
    else if (bkc) hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_BF16, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<TL, DT_BF16, false, false>), grid, block, 0, s, a);
  }
}

template void launch_pipelined<Tile256D>(GemmArgs, int, int, int, hipStream_t);

}  // namespace trt
