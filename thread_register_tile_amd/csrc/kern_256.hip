// kern_256.hip -- generic-kernel instances of one tile (256x256x64).
#include "kern_generic.hpp"

namespace trt {

template hipError_t launch_generic<Tile256>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
