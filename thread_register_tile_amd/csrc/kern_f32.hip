// kern_f32.hip -- instances of the binary32-operand GEMM.
#include "gemm_f32.hpp"
#include "gemm_f32_dma.hpp"
#include "tiles.hpp"

namespace trt {

void launch_f32(GemmArgs a, int opA, int opB, bool vec, hipStream_t s) {
  a.tiles_m = (a.M + TileF32::BM - 1) / TileF32::BM;
  a.tiles_n = (a.N + TileF32::BN - 1) / TileF32::BN;
  const dim3 grid(a.tiles_m * a.tiles_n), block(256);
  const bool akc = opA == 0, bkc = opB == 1;
  // direct-to-LDS copies: aligned 16-byte rows, no chunk straddling an
  // operand's end, extents addressable by 32-bit offsets
  const bool dma = vec && (akc ? a.K % 4 == 0 : a.M % 4 == 0) &&
                   (bkc ? a.K % 4 == 0 : a.N % 4 == 0) && a.a_bytes < (int64_t(1) << 31) &&
                   a.b_bytes < (int64_t(1) << 31);
  if (dma) {
    if (akc && bkc) hipLaunchKernelGGL((gemm_f32_dma_kernel<true, true>), grid, block, 0, s, a);
    else if (akc) hipLaunchKernelGGL((gemm_f32_dma_kernel<true, false>), grid, block, 0, s, a);
    else if (bkc) hipLaunchKernelGGL((gemm_f32_dma_kernel<false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_f32_dma_kernel<false, false>), grid, block, 0, s, a);
    return;
  }
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
