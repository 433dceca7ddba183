// kern_f32.hip -- instances of the binary32-operand GEMM.
#include "gemm_f32.hpp"
#include "tiles.hpp"

namespace trt {

void launch_f32(GemmArgs a, int opA, int opB, bool vec, hipStream_t s) {
  a.tiles_m = (a.M + TileF32::BM - 1) / TileF32::BM;
  a.tiles_n = (a.N + TileF32::BN - 1) / TileF32::BN;
  const dim3 grid(a.tiles_m * a.tiles_n), block(256);
  const bool akc = opA == 0, bkc = opB == 1;
#define TRT_F32_LAUNCH(AK, BK, V) \
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BK, V>), grid, block, 0, s, a)
  if (vec) {
    if (akc && bkc) TRT_F32_LAUNCH(true, true, true);
    else if (akc) TRT_F32_LAUNCH(true, false, true);
    else if (bkc) TRT_F32_LAUNCH(false, true, true);
    else TRT_F32_LAUNCH(false, false, true);
  } else {
    if (akc && bkc) TRT_F32_LAUNCH(true, true, false);
    else if (akc) TRT_F32_LAUNCH(true, false, false);
    else if (bkc) TRT_F32_LAUNCH(false, true, false);
    else TRT_F32_LAUNCH(false, false, false);
  }
#undef TRT_F32_LAUNCH
}

}  // namespace trt
