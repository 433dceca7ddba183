// kern_tiny.hip -- generic-kernel instances of one tile (16x64x32, one wave: the named GEMM's tile).
#include "kern_generic.hpp"

namespace trt {

template hipError_t launch_generic<TileTiny>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
