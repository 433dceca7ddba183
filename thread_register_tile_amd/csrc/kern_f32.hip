// kern_f32.hip -- instances of the binary32-operand GEMM.
#include "gemm_f32.hpp"
#include "gemm_f32_dma.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

namespace {

template <bool AK, bool BK>
hipError_t launch_f32_ops(const GemmArgs& a, bool dma, bool vec, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (dma) return launch(gemm_f32_dma_kernel<AK, BK>, grid, block, 0, s, a);
  if (vec) return launch(gemm_f32_kernel<AK, BK, true>, grid, block, 0, s, a);
  return launch(gemm_f32_kernel<AK, BK, false>, grid, block, 0, s, a);
}

}  // namespace

hipError_t launch_f32(GemmArgs a, int opA, int opB, bool vec, hipStream_t s) {
  a.tiles_m = (a.M + TileF32::BM - 1) / TileF32::BM;
  a.tiles_n = (a.N + TileF32::BN - 1) / TileF32::BN;
  const dim3 grid(a.tiles_m * a.tiles_n);
  const bool akc = opA == 0, bkc = opB == 1;
  // direct-to-LDS copies: aligned 16-byte rows, no chunk straddling an
  // operand's end, extents addressable by 32-bit offsets, and rows-
  // contiguous operands whose rows do not overlap (ld at least the row
  // length), so that the rows k >= K of a partial last K step lie past the
  // operand's end and read as zero
  const bool dma = vec && (akc ? a.K % 4 == 0 : a.M % 4 == 0 && a.lda >= a.M) &&
                   (bkc ? a.K % 4 == 0 : a.N % 4 == 0 && a.ldb >= a.N) &&
                   a.a_bytes < (int64_t(1) << 31) && a.b_bytes < (int64_t(1) << 31);
  if (akc && bkc) return launch_f32_ops<true, true>(a, dma, vec, grid, s);
  if (akc) return launch_f32_ops<true, false>(a, dma, vec, grid, s);
  if (bkc) return launch_f32_ops<false, true>(a, dma, vec, grid, s);
  return launch_f32_ops<false, false>(a, dma, vec, grid, s);
}

}  // namespace trt
