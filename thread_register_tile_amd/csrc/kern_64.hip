// kern_64.hip -- generic-kernel instances of one tile (64x64x64).
#include "kern_generic.hpp"

namespace trt {

template hipError_t launch_generic<Tile64>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
