// kern_dma256_f16_ak.hip -- instances of the pipelined direct-to-LDS
// kernel (256x256 tile of 8 waves, K step 32, 16x16x32 fragments) for f16 inputs with
// A stored k-contiguous, in a translation unit of their own so that the
// library builds in parallel.
#include "kern_pipelined.hpp"

namespace trt {

template hipError_t launch_pipelined_a<Tile256D, DT_F16, true>(GemmArgs, bool, hipStream_t);

}  // namespace trt
