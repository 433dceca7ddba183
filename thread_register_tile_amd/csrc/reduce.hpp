// reduce.hpp -- the rank-1 block reduction for gfx950.
//
// "My Triton From Scratch, Part 12: CUDA Tile Layouts", section "Output shape
// is not always thread shape": a program instance reduces a block of BLOCK
// consecutive elements to one stored scalar (sum, maximum or minimum); its
// output tile is (1,) but the reduction needs BLOCK-wide cooperation.  Here a
// block is reduced by W wavefronts (W = 1 for small blocks, 4 for large
// ones): the block's elements are dealt to the W*64 lanes as 16-byte chunks
// in the cooperative order of the same page ("Cooperative tile layouts":
// chunk c of the block goes to lane c mod 64W, iteration c div 64W), each
// lane folds its chunks in fp32, the wave folds its lanes with cross-lane
// shuffles, and W > 1 waves meet in LDS.  A workgroup of 4 waves reduces 4/W
// blocks at a time and walks the grid of blocks in strides.
//
// The last block may be shorter than BLOCK: its missing elements are masked
// off.  Inputs are f16, bf16 or f32; the result is f32.  Maximum and minimum
// are NaN when any element of the block is NaN; a sum with a NaN is NaN.
#pragma once

#include "gemm_kernel.hpp"

namespace trt {

enum : int { RED_SUM = 0, RED_MAX = 1, RED_MIN = 2 };

struct ReduceArgs {
  const void* x;
  float* out;
  int64_t n;         // elements
  int64_t block;     // elements per block
  int64_t nblocks;   // ceil(n / block)
  int32_t vec;       // 16-byte chunks allowed: x 16-byte aligned, block * element size % 16 == 0
};

template <int DT>
struct RedIn {
  static constexpr int VEC = 8;  // elements per 16-byte chunk
  __device__ static float ld(const void* p, int64_t i) {
    return to_f32<DT>(static_cast<const uint16_t*>(p)[i]);
  }
  template <class F>
  __device__ static void chunk(const void* p, int64_t i, F&& f) {
    const u32x4 w = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f(to_f32<DT>(w[q] & 0xFFFFu));
      f(to_f32<DT>(w[q] >> 16));
    }
  }
};
template <>
struct RedIn<DT_F32> {
  static constexpr int VEC = 4;
  __device__ static float ld(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  template <class F>
  __device__ static void chunk(const void* p, int64_t i, F&& f) {
    const f32x4 w = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i));
#pragma unroll
    for (int q = 0; q < 4; ++q) f(w[q]);
  }
};

template <int OP>
__device__ __forceinline__ float red_identity() {
  return OP == RED_SUM ? 0.f : (OP == RED_MAX ? -__builtin_inff() : __builtin_inff());
}

template <int OP>
__device__ __forceinline__ float red_op(float a, float b) {
  if (OP == RED_SUM) return a + b;
  return OP == RED_MAX ? __builtin_fmaxf(a, b) : __builtin_fminf(a, b);
}

template <int DT, int OP, int W>
__global__ __launch_bounds__(256) void block_reduce_kernel(ReduceArgs a) {
  using I = RedIn<DT>;
  constexpr int VEC = I::VEC;
  constexpr int GROUPS = 4 / W;             // blocks reduced at a time per workgroup
  constexpr int LANES = 64 * W;             // lanes per block
  __shared__ float part[4];
  __shared__ int part_nan[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = wave / W, wv = wave % W;
  const int me = 64 * wv + lane;            // this lane's place among the block's lanes
  for (int64_t b = (int64_t)blockIdx.x * GROUPS + grp; b - grp < a.nblocks;
       b += (int64_t)gridDim.x * GROUPS) {
    const bool live = b < a.nblocks;        // uniform per wave: every wave runs every trip
    const int64_t e0 = b * a.block;
    const int64_t len = live ? (a.n - e0 < a.block ? a.n - e0 : a.block) : 0;
    float acc = red_identity<OP>();
    bool nan = false;
    auto fold = [&](float v) {
      if (OP != RED_SUM) nan |= v != v;
      acc = red_op<OP>(acc, v);
    };
    // whole 16-byte chunks, four in flight per lane
    const int64_t chunks = a.vec ? len / VEC : 0;
    int64_t c = me;
    for (; c + 3 * LANES < chunks; c += 4 * LANES) {
#pragma unroll
      for (int u = 0; u < 4; ++u) I::chunk(a.x, e0 + VEC * (c + u * LANES), fold);
    }
    for (; c < chunks; c += LANES) I::chunk(a.x, e0 + VEC * c, fold);
    // the rest element by element (the tail, or everything without chunks)
    for (int64_t e = VEC * chunks + me; e < len; e += LANES) fold(I::ld(a.x, e0 + e));
    // fold the wave's 64 lanes
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc = red_op<OP>(acc, __shfl_xor(acc, off));
    const bool wave_nan = __any(nan);
    if (W == 1) {
      if (live && lane == 0) a.out[b] = wave_nan ? __builtin_nanf("") : acc;
    } else {
      if (lane == 0) {
        part[wave] = acc;
        part_nan[wave] = wave_nan;
      }
      __syncthreads();
      if (live && t == 0) {
        float r = part[0];
        bool any_nan = part_nan[0];
#pragma unroll
        for (int w = 1; w < W; ++w) {
          r = red_op<OP>(r, part[w]);
          any_nan |= part_nan[w] != 0;
        }
        a.out[b] = any_nan ? __builtin_nanf("") : r;
      }
      __syncthreads();
    }
  }
}

}  // namespace trt
