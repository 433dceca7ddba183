// kern_128.hip -- generic-kernel instances of one tile (128x128x64), compiled as a
// translation unit of its own so that the library builds in parallel.
#include "gemm_kernel.hpp"
#include "tiles.hpp"

namespace trt {

template <class TL, int DT, bool AKC, bool BKC>
static void launch_vec(const GemmArgs& a, bool vec, dim3 grid, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((gemm_kernel<TL, DT, AKC, BKC, true>), grid, dim3(TL::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<TL, DT, AKC, BKC, false>), grid, dim3(TL::THREADS), 0, s, a);
}

template <class TL, int DT>
static void launch_ops(const GemmArgs& a, int opA, int opB, bool vec, dim3 grid, hipStream_t s) {
  const bool akc = opA == 0, bkc = opB == 1;
  if (akc && bkc) launch_vec<TL, DT, true, true>(a, vec, grid, s);
  else if (akc) launch_vec<TL, DT, true, false>(a, vec, grid, s);
  else if (bkc) launch_vec<TL, DT, false, true>(a, vec, grid, s);
  else launch_vec<TL, DT, false, false>(a, vec, grid, s);
}

template <class TL>
void launch_generic(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s) {
  a.tiles_m = (a.M + TL::BM - 1) / TL::BM;
  a.tiles_n = (a.N + TL::BN - 1) / TL::BN;
  const dim3 grid(a.tiles_m * a.tiles_n);
  if (dt == DT_F16) launch_ops<TL, DT_F16>(a, opA, opB, vec, grid, s);
  else launch_ops<TL, DT_BF16>(a, opA, opB, vec, grid, s);
}

template void launch_generic<Tile128>(GemmArgs, int, int, int, bool, hipStream_t);

}  // namespace trt
