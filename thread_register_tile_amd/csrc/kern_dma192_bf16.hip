// kern_dma192_bf16.hip -- instances of the pipelined direct-to-LDS kernel on
// the 256x192 tile (8x6 fragments of 16x16 per wave: a register tile that is
// not a power of two) for bf16 inputs, in a translation unit of their own.
#include "kern_pipelined.hpp"

namespace trt {

template hipError_t launch_pipelined_a<Tile256x192D, DT_BF16, true>(GemmArgs, bool, hipStream_t);
template hipError_t launch_pipelined_a<Tile256x192D, DT_BF16, false>(GemmArgs, bool, hipStream_t);

}  // namespace trt
