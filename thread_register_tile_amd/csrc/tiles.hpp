// tiles.hpp -- the compiled workgroup tiles and their launch entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace trt {

using TileTiny = Tile<16, 64, 32, 1, 1>;       // one wave, the named GEMM's tile
using Tile64 = Tile<64, 64, 64, 2, 2>;         // 4 waves, 32x32 each
using Tile128 = Tile<128, 128, 64, 2, 2>;      // 4 waves, 64x64 each
using Tile256 = Tile<256, 256, 64, 2, 2>;      // 4 waves, 128x128 each
using Tile256D = Tile<256, 256, 32, 2, 4, 16>; // pipelined, 8 waves of 8x4 fragments of 16x16
using Tile256x192D = Tile<256, 192, 32, 2, 2, 16>;  // pipelined, 8x6 fragments of 16x16 per wave
using Tile256F = Tile<256, 256, 32, 2, 2, 16>; // generic kernel on the pipelined tile
using Tile128D = Tile<128, 128, 32, 2, 2, 16>; // pipelined, 4 waves of 4x4 fragments of 16x16

// Every launch function returns the runtime's status of its own launch.

// Launch the generic kernel of tile TL (defined in kern_generic.hpp, and
// explicitly instantiated per tile in the kern_*.hip translation units).
template <class TL>
hipError_t launch_generic(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s);

// Launch the pipelined direct-to-LDS kernel of tile TL for input type DT and
// A storage (A_KC: k-contiguous), defined in kern_pipelined.hpp and
// instantiated per (tile, DT, A storage) in the kern_dma*.hip units.
template <class TL, int DT, bool A_KC>
hipError_t launch_pipelined_a(GemmArgs a, bool b_kc, hipStream_t s);

template <class TL>
inline hipError_t launch_pipelined(GemmArgs a, int dt, int opA, int opB, hipStream_t s) {
  a.tiles_m = (a.M + TL::BM - 1) / TL::BM;
  a.tiles_n = (a.N + TL::BN - 1) / TL::BN;
  const bool akc = opA == 0, bkc = opB == 1;
  if (dt == DT_F16)
    return akc ? launch_pipelined_a<TL, DT_F16, true>(a, bkc, s)
               : launch_pipelined_a<TL, DT_F16, false>(a, bkc, s);
  return akc ? launch_pipelined_a<TL, DT_BF16, true>(a, bkc, s)
             : launch_pipelined_a<TL, DT_BF16, false>(a, bkc, s);
}

// Launch the HBM-streaming kernel for M <= 16 (kern_skinny.hip).
hipError_t launch_skinny(GemmArgs a, int dt, hipStream_t s);

// Launch the split-K streaming kernel for M <= 16 (`splits` K slices of
// `per_split` iterations of 32 k, partials in the workspace ws) and the
// reduction that adds them and applies the epilogue (kern_skinny.hip).
hipError_t launch_skinny_split(GemmArgs a, int dt, float* ws, int splits, int per_split,
                               hipStream_t s);

// Launch the binary32-operand GEMM on its 128x128x32 tile (kern_f32.hip).
hipError_t launch_f32(GemmArgs a, int opA, int opB, bool vec, hipStream_t s);

// Launch the register-tile GEMM on vector lanes (kern_regtile.hip).
struct RegtileArgs;
hipError_t launch_regtile(RegtileArgs a, int dt, hipStream_t s);

// Launch the rank-1 block reduction (kern_reduce.hip).
struct ReduceArgs;
hipError_t launch_reduce(const ReduceArgs& a, int dt, int op, hipStream_t s);

}  // namespace trt
