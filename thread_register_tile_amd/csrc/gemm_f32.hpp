// gemm_f32.hpp -- the GEMM on binary32 operands for gfx950.
//
// The pages' register-tile GEMM computes in f32 on general-purpose lanes ("My
// Triton From Scratch, Part 16: Register Tiles", section "What Version 16
// does not optimize"); on gfx950 binary32 products run on the matrix cores as
// v_mfma_f32_16x16x4_f32.  Workgroup tile 128x128 with a K step of 32, 2x2
// waves of 64x64, 4x4 fragments of 16x16: the ownership map and the fused
// epilogue are those of the generic kernel's 16x16 tiles (Tile<128, 128, 32,
// 2, 2, 16>), so it reuses epilogue_store.
//
// Both operand tiles are staged k-contiguous in LDS, A as [128 m][32 k] and
// B as [128 n][32 k], rows of 32 floats (eight 16-byte chunks) with chunk kc
// of row r stored at chunk kc ^ sw(r), sw(r) = (r ^ (r >> 3)) & 7.
// Matrix-core step kk (0..7) of a K step takes k = 8*(lane/16) + kk: each
// lane reads its 8 k of a fragment row as two 16-byte LDS loads.  LDS serves
// a 16-byte-per-lane access eight lanes at a time, each group of eight from
// one 128-byte bank window: eight consecutive rows of one chunk sit at eight
// distinct positions of their rows (sw takes row bits 0-2), so the fragment
// reads are conflict-free (a swizzle on row bits 1-3 put row pairs on one
// position and read 16.8 M conflict cycles per 4096^3 launch).  Storage with
// k contiguous in global memory is copied as 16-byte chunks (row c/8, chunk
// c%8: eight lanes fill one row).  Storage with m (or n) contiguous is read
// as a 4x4 block per thread -- four k rows of four consecutive m, the 32
// lanes of a half-wave covering 512 contiguous bytes of one k row --
// transposed in registers and written as four k-contiguous chunks, eight
// lanes on rows 4 apart, at distinct positions.  Out-of-range rows and k
// are zero.
#pragma once

#include "gemm_kernel.hpp"

namespace trt {

using TileF32 = Tile<128, 128, 32, 2, 2, 16>;

__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int f32_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Float offset of chunk kc (4 floats of k) of LDS row r.
__device__ __forceinline__ int f32_slot(int r, int kc) { return r * 32 + 4 * (kc ^ f32_swz(r)); }

// One operand's copy: 128 rows (m or n) x 32 k per K step, four 16-byte
// chunks per thread.  KC: k contiguous in global memory (element (r, k) at
// X[r*ld + k]); else (r, k) at X[k*ld + r].
template <bool KC, bool VEC>
struct F32Operand {
  static constexpr int R = 128;
  f32x4 v[4];

  __device__ __forceinline__ void load(const float* X, int64_t ld, int r0, int rows, int k0,
                                       int K, int t, bool full) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // KC: chunk c = (row c/8, k 4*(c%8)..+3); else k row 4*(t/32) + i,
      // rows 4*(t%32)..+3
      const int c = t + 256 * i;
      const int r = KC ? c / 8 : 4 * (t % 32);
      const int k = KC ? 4 * (c % 8) : 4 * (t / 32) + i;
      const int64_t base = KC ? (int64_t)(r0 + r) * ld + k0 + k : (int64_t)(k0 + k) * ld + r0 + r;
      if (VEC && full) {
        v[i] = *reinterpret_cast<const f32x4*>(X + base);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = KC ? (r0 + r < rows && k0 + k + e < K) : (r0 + r + e < rows && k0 + k < K);
          v[i][e] = ok ? X[base + e] : 0.f;
        }
      }
    }
  }

  __device__ __forceinline__ void store(float* lds, int t) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (KC) {
        const int c = t + 256 * i;
        *reinterpret_cast<f32x4*>(lds + f32_slot(c / 8, c % 8)) = v[i];
      } else {
        // row 4*(t%32) + i of the block: element i of each of the four k rows
        const int r = 4 * (t % 32) + i;
        const f32x4 w = {v[0][i], v[1][i], v[2][i], v[3][i]};
        *reinterpret_cast<f32x4*>(lds + f32_slot(r, t / 32)) = w;
      }
    }
  }
};

template <bool A_KC, bool B_KC, bool VEC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  using TL = TileF32;
  constexpr int BM = TL::BM, BN = TL::BN, FM = TL::FM, FN = TL::FN;
  static_assert(FM == 4 && FN == 4 && TL::THREADS == 256, "2x2 waves of 4x4 fragments");
  __shared__ __attribute__((aligned(16))) float lds[2][(BM + BN) * 32];
  const float* A = reinterpret_cast<const float*>(p.A);
  const float* B = reinterpret_cast<const float*>(p.B);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int tm, tn;
  tile_of<8>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const bool full_mn = (m0 + BM <= p.M) && (n0 + BN <= p.N);

  static_assert(BM == F32Operand<true, true>::R && BN == F32Operand<true, true>::R, "128-row operands");
  F32Operand<A_KC, VEC> a;
  F32Operand<B_KC, VEC> b;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (p.K + 31) / 32;
  auto load_step = [&](int kt) {
    const int k0 = kt * 32;
    const bool full = full_mn && k0 + 32 <= p.K;
    a.load(A, p.lda, m0, p.M, k0, p.K, t, full);
    b.load(B, p.ldb, n0, p.N, k0, p.K, t, full);
  };
  const int wrow = (wave / TL::WN) * TL::WTM, wcol = (wave % TL::WN) * TL::WTN;
  const int fr = lane & 15, g = lane >> 4;

  // One K step: the first half's fragments are read, the next step's copy is
  // issued, then the first half's 64 products run with the second half's
  // fragment reads interleaved, and the second half's 64 products with the
  // next step's LDS writes interleaved (the other buffer was last read
  // before the previous barrier).  Scheduling groups fix the interleave.
  auto frag = [&](const float* base, int row, int h) {
    return *reinterpret_cast<const f32x4*>(base + f32_slot(row, 2 * g + h));
  };
  load_step(0);
  a.store(lds[0], t);
  b.store(lds[0] + BM * 32, t);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const float* la = lds[cur];
    const float* lb = lds[cur] + BM * 32;
    f32x4 af[FM][2], bf[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i][0] = frag(la, wrow + 16 * i + fr, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j][0] = frag(lb, wcol + 16 * j + fr, 0);
    if (more) load_step(kt + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i][1] = frag(la, wrow + 16 * i + fr, 1);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j][1] = frag(lb, wcol + 16 * j + fr, 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16_f32(bf[j][0][kk], af[i][0][kk], acc[i][j]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 32, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      a.store(lds[cur ^ 1], t);
      b.store(lds[cur ^ 1] + BM * 32, t);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16_f32(bf[j][1][kk], af[i][1][kk], acc[i][j]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 2, 0);   // register transposes
      __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 32, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }
  epilogue_store<TL>(p, acc, m0, n0, lane, wave);
}

}  // namespace trt
