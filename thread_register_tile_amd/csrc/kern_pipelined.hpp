// kern_pipelined.hpp -- the launcher of the pipelined direct-to-LDS kernel,
// included only by the kern_dma*.hip units, each of which instantiates it
// for one tile and input type (the library builds them in parallel).
#pragma once

#include "gemm_dma.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

template <class TL, int DT, bool A_KC>
hipError_t launch_pipelined_a(GemmArgs a, bool b_kc, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n);
  const dim3 block(TL::THREADS);
  if (b_kc) return launch(gemm_dma_kernel<TL, DT, A_KC, true>, grid, block, 0, s, a);
  return launch(gemm_dma_kernel<TL, DT, A_KC, false>, grid, block, 0, s, a);
}

}  // namespace trt
