// kern_128.hip -- generic-kernel instances of one tile (128x128x64).
#include "kern_generic.hpp"

namespace trt {

template hipError_t launch_generic<Tile128>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
