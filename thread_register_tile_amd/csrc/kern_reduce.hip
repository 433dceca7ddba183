// kern_reduce.hip -- instances of the rank-1 block reduction.
#include "reduce.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

namespace {

template <int DT, int OP>
hipError_t launch_dt_op(const ReduceArgs& a, hipStream_t s) {
  // a block of at least 8192 elements keeps four waves busy; smaller ones
  // take one wave each, four blocks per workgroup
  const bool wide = a.block >= 8192;
  const int64_t groups = wide ? 1 : 4;
  int64_t wgs = (a.nblocks + groups - 1) / groups;
  if (wgs > 16384) wgs = 16384;               // grid-stride beyond this
  const dim3 grid((unsigned)wgs), block(256);
  if (wide) return launch(block_reduce_kernel<DT, OP, 4>, grid, block, 0, s, a);
  return launch(block_reduce_kernel<DT, OP, 1>, grid, block, 0, s, a);
}

template <int DT>
hipError_t launch_dt(const ReduceArgs& a, int op, hipStream_t s) {
  if (op == RED_SUM) return launch_dt_op<DT, RED_SUM>(a, s);
  if (op == RED_MAX) return launch_dt_op<DT, RED_MAX>(a, s);
  return launch_dt_op<DT, RED_MIN>(a, s);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dt, int op, hipStream_t s) {
  if (dt == DT_F16) return launch_dt<DT_F16>(a, op, s);
  if (dt == DT_BF16) return launch_dt<DT_BF16>(a, op, s);
  return launch_dt<DT_F32>(a, op, s);
}

}  // namespace trt
