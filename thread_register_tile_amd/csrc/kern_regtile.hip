// kern_regtile.hip -- instances of the register-tile GEMM on vector lanes:
// three input types x register bounds {1, 2, 4, 8} per axis.
#include "regtile.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace trt {

namespace {

int reg_bound(int r) { return r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : 8; }

template <int DT, int MRM, int MRN>
hipError_t launch_pf(const RegtileArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  if (a.prefetch)
    return launch(gemm_regtile_kernel<DT, MRM, MRN, true>, grid, dim3(kRegtileThreads), lds, s, a);
  return launch(gemm_regtile_kernel<DT, MRM, MRN, false>, grid, dim3(kRegtileThreads), lds, s, a);
}

template <int DT, int MRM>
hipError_t launch_rn(const RegtileArgs& a, int mrn, dim3 grid, size_t lds, hipStream_t s) {
  switch (mrn) {
    case 1: return launch_pf<DT, MRM, 1>(a, grid, lds, s);
    case 2: return launch_pf<DT, MRM, 2>(a, grid, lds, s);
    case 4: return launch_pf<DT, MRM, 4>(a, grid, lds, s);
    default: return launch_pf<DT, MRM, 8>(a, grid, lds, s);
  }
}

template <int DT>
hipError_t launch_dt(const RegtileArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const int mrm = reg_bound(a.rm), mrn = reg_bound(a.rn);
  switch (mrm) {
    case 1: return launch_rn<DT, 1>(a, mrn, grid, lds, s);
    case 2: return launch_rn<DT, 2>(a, mrn, grid, lds, s);
    case 4: return launch_rn<DT, 4>(a, mrn, grid, lds, s);
    default: return launch_rn<DT, 8>(a, mrn, grid, lds, s);
  }
}

}  // namespace

hipError_t launch_regtile(RegtileArgs a, int dt, hipStream_t s) {
  a.g.tiles_m = (int)((a.g.M + a.lm - 1) / a.lm);
  a.g.tiles_n = (int)((a.g.N + a.ln - 1) / a.ln);
  const dim3 grid((unsigned)((int64_t)a.g.tiles_m * a.g.tiles_n));
  // both operand tiles, then one float that masked-off copies write to
  const size_t lds = sizeof(float) * (kRegtilePitch * (a.lm + a.ln) + 1);
  // at most kRegtilePF elements of each operand tile per lane, operands
  // addressable by 32-bit byte offsets
  a.prefetch = (a.lm * kRegtileBK + kRegtileThreads - 1) / kRegtileThreads <= kRegtilePF &&
               (a.ln * kRegtileBK + kRegtileThreads - 1) / kRegtileThreads <= kRegtilePF &&
               a.g.a_bytes < (int64_t(1) << 31) && a.g.b_bytes < (int64_t(1) << 31);
  if (dt == DT_F16) return launch_dt<DT_F16>(a, grid, lds, s);
  if (dt == DT_BF16) return launch_dt<DT_BF16>(a, grid, lds, s);
  return launch_dt<DT_F32>(a, grid, lds, s);
}

}  // namespace trt
