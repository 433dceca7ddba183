// kern_dma128.hip -- instances of the pipelined kernel on the 128x128x32 tile
// (4 waves of 4x4 fragments of 16x16, two workgroups per compute unit), for
// problems too small to give every compute unit a 256-wide tile.
#include "kern_pipelined.hpp"

namespace trt {

template hipError_t launch_pipelined_a<Tile128D, DT_F16, true>(GemmArgs, bool, hipStream_t);
template hipError_t launch_pipelined_a<Tile128D, DT_F16, false>(GemmArgs, bool, hipStream_t);
template hipError_t launch_pipelined_a<Tile128D, DT_BF16, true>(GemmArgs, bool, hipStream_t);
template hipError_t launch_pipelined_a<Tile128D, DT_BF16, false>(GemmArgs, bool, hipStream_t);

}  // namespace trt
