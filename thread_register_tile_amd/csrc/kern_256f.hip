// kern_256f.hip -- generic-kernel instances of one tile (256x256x32 with 16x16x32 fragments: the pipelined tile's fallback).
#include "kern_generic.hpp"

namespace trt {

template hipError_t launch_generic<Tile256F>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
