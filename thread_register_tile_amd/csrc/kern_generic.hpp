// kern_generic.hpp -- the launcher of the generic register-tile kernel,
// included only by the kern_*.hip units that instantiate it, one tile per
// translation unit so that the library builds in parallel.
#pragma once

#include "gemm_kernel.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

template <class TL, int DT, bool AKC, bool BKC>
hipError_t launch_generic_vec(const GemmArgs& a, bool vec, dim3 grid, hipStream_t s) {
  if (vec) return launch(gemm_kernel<TL, DT, AKC, BKC, true>, grid, dim3(TL::THREADS), 0, s, a);
  return launch(gemm_kernel<TL, DT, AKC, BKC, false>, grid, dim3(TL::THREADS), 0, s, a);
}

template <class TL, int DT>
hipError_t launch_generic_ops(const GemmArgs& a, int opA, int opB, bool vec, dim3 grid,
                              hipStream_t s) {
  const bool akc = opA == 0, bkc = opB == 1;
  if (akc && bkc) return launch_generic_vec<TL, DT, true, true>(a, vec, grid, s);
  if (akc) return launch_generic_vec<TL, DT, true, false>(a, vec, grid, s);
  if (bkc) return launch_generic_vec<TL, DT, false, true>(a, vec, grid, s);
  return launch_generic_vec<TL, DT, false, false>(a, vec, grid, s);
}

template <class TL>
hipError_t launch_generic(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s) {
  a.tiles_m = (a.M + TL::BM - 1) / TL::BM;
  a.tiles_n = (a.N + TL::BN - 1) / TL::BN;
  const dim3 grid(a.tiles_m * a.tiles_n);
  if (dt == DT_F16) return launch_generic_ops<TL, DT_F16>(a, opA, opB, vec, grid, s);
  return launch_generic_ops<TL, DT_BF16>(a, opA, opB, vec, grid, s);
}

}  // namespace trt
