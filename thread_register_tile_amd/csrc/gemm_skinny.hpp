// gemm_skinny.hpp -- the GEMM for M <= 16: a pure stream over B.
//
// With at most 16 rows of A, each element of B is used by at most 16
// products: the operation is bound by reading B from HBM once.  One
// workgroup owns a 64-column panel of C ([16, 64], the tile of the NineToothed
// "Named layouts" GEMM arrangement) and all of K.  Its 8 waves split K between
// them; each wave streams its slice of the panel straight from global memory
// into registers -- no LDS on the way -- keeping DEPTH iterations of loads in
// flight, and accumulates a partial [16, 64] tile on the 16x16x32 matrix
// cores.  The 8 partial tiles are summed through LDS in a fixed order
// (deterministic, no atomics) and the fused epilogue stores the panel.
//
// One iteration of a wave covers 32 k x 64 columns of B: lane l loads 8 bytes
// (4 columns, n = 4*(l%16)) of the 8 k rows 8*(l/16) .. 8*(l/16)+7, and
// transposes the 8 x 4 block in registers into four operand registers of 8
// k values, one per column n + j.  Product j then covers the 16 columns
// {4i + j : i = 0..15} (operand column i is lane l%16 = i).  A's operand (16
// rows, 8 consecutive k per lane) is one 16-byte load.
//
// Requirements (checked by the dispatcher): A stored k-contiguous and B
// row-major; 16-byte aligned A rows (lda % 8 == 0), 8-byte aligned B rows
// (ldb % 4 == 0); K % 8 == 0 and N % 4 == 0, so that every vector load is
// wholly inside or outside the operand.  Loads outside are redirected to the
// operand's first element and their values replaced by zero.
#pragma once

#include "gemm_kernel.hpp"

namespace trt {

// The workgroup tile of the skinny kernel: logical [16, 64], 8 waves, and
// after the cross-wave reduction every thread owns 2 consecutive columns of
// one row: thread t = 64*wave + lane holds C(t / 32, 2*(t % 32) + reg).
struct SkinnyTile {
  static constexpr int BM = 16, BN = 64, WAVES = 8, THREADS = 64 * WAVES;
  static constexpr int KW = 32;      // k per wave iteration
  static constexpr int DEPTH = 4;    // iterations of loads in flight per wave
  static constexpr int REGS = 2;     // outputs per thread after the reduction
  TRT_HD static int owner_row(int reg, int lane, int wave) { return (64 * wave + lane) / 32; }
  TRT_HD static int owner_col(int reg, int lane, int wave) {
    return 2 * ((64 * wave + lane) % 32) + reg;
  }
  static constexpr int REG_BITS = 1, WAVE_BITS = 3, C_IN_BITS = REG_BITS + 6 + WAVE_BITS;
  static constexpr Gf2Map<C_IN_BITS> c_map() {
    Gf2Map<C_IN_BITS> m{};
    m.row_bits = 4;
    m.col_bits = 6;
    int i = 0;
    m.b[i++] = {0, 1};                                   // reg
    for (int s = 0; s < 5; ++s) m.b[i++] = {0, 2 << s};  // lane bits 0-4
    m.b[i++] = {1, 0};                                   // lane bit 5
    for (int s = 0; s < 3; ++s) m.b[i++] = {2 << s, 0};  // wave bits
    return m;
  }
  static constexpr bool owner_matches_bases() {
    constexpr auto m = c_map();
    for (int w = 0; w < WAVES; ++w)
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < REGS; ++r) {
          const Basis v = m.apply(uint32_t(r) | (uint32_t(l) << 1) | (uint32_t(w) << 7));
          if (v.row != owner_row(r, l, w) || v.col != owner_col(r, l, w)) return false;
        }
    return true;
  }
};
static_assert(SkinnyTile::c_map().bijective(), "C ownership must cover the tile exactly once");

// One wave's stream over B: its 64 columns n0 .. n0+63 of B, iterations
// it0 .. it1-1 of 32 k, accumulated into acc[j] (register r of acc[j] is
// row 4*(lane/16) + r, column 4*(lane%16) + j of the 64).
template <int DT>
__device__ __forceinline__ void skinny_stream(const GemmArgs& p, int n0, int it0, int it1,
                                              int lane, f32x4 (&acc)[4]) {
  using ST = SkinnyTile;
  constexpr int D = ST::DEPTH;
  const int c = lane & 15, g = lane >> 4;
  const int n = n0 + 4 * c;                 // this lane's 4 columns of B
  const int ma = lane & 15;                 // this lane's row of A
  const int iters = max(it1 - it0, 0);

  u32x2 bq[D][8];
  u32x4 aq[D];
  // Loads of iteration `it` (absolute) into slot s.
  auto load = [&](int it, int s) {
    const int kb = it * ST::KW + 8 * g;
    const bool a_ok = ma < p.M && kb < p.K;
    const u32x4 av = *reinterpret_cast<const u32x4*>(p.A + (a_ok ? (int64_t)ma * p.lda + kb : 0));
    aq[s] = a_ok ? av : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = n < p.N && kb + j < p.K;
      // B is read exactly once: non-temporal loads keep it from displacing
      // cache lines that are reused
      const u32x2 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(p.B + (ok ? (int64_t)(kb + j) * p.ldb + n : 0)));
      bq[s][j] = ok ? v : u32x2{0u, 0u};
    }
  };

#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto consume = [&](int s) {
    // 8 k rows x 4 columns -> 4 operand registers of 8 k each
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = j >> 1;
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __builtin_amdgcn_perm(bq[s][2 * q + 1][w], bq[s][2 * q][w], sel);
      acc[j] = mfma16<DT>(aq[s], f, acc[j]);
    }
  };

#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < iters) load(it0 + s, s);
  int i = 0;
  for (; i + D <= iters; i += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      consume(s);
      if (i + D + s < iters) load(it0 + i + D + s, s);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (i + s < iters) consume(s);
}

template <int DT>
__global__ __launch_bounds__(SkinnyTile::THREADS) void gemm_skinny_kernel(GemmArgs p) {
  using ST = SkinnyTile;
  __shared__ f32x4 part[ST::WAVES][4][64];  // partial tiles: [wave][j][lane]

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * ST::BN;

  // the wave's K slice, in whole iterations of 32
  const int iters_total = (p.K + ST::KW - 1) / ST::KW;
  const int per_wave = (iters_total + ST::WAVES - 1) / ST::WAVES;
  const int it0 = wave * per_wave;
  const int it1 = min(it0 + per_wave, iters_total);

  f32x4 acc[4];
  skinny_stream<DT>(p, n0, it0, it1, lane, acc);

  // cross-wave reduction: partial (m, n) of wave w sits at part[w][j][lane]
  // register r with m = 4*(lane/16) + r, n = 4*(lane%16) + j
#pragma unroll
  for (int j = 0; j < 4; ++j) part[wave][j][lane] = acc[j];
  __syncthreads();

  const int m = ST::owner_row(0, lane, wave);
  const int nl = ST::owner_col(0, lane, wave);  // columns nl, nl + 1
  float y[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int ncol = nl + e;
    const int j = ncol & 3, src_lane = 16 * (m >> 2) + (ncol >> 2), r = m & 3;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < ST::WAVES; ++w) sum += part[w][j][src_lane][r];
    y[e] = sum;
  }
  if (m >= p.M) return;
  const int nc = n0 + nl;
  with_out_type(p.out_dt, [&]<int OT>() {
    using O = Out<OT>;
    const float s = p.scale ? O::ld(p.scale, m) : 1.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (nc + e >= p.N) continue;
      float v = y[e];
      if (p.scale) v *= s;
      if (p.bias) v += O::ld(p.bias, nc + e);
      if (p.relu) v = v > 0.f ? v : 0.f;
      if (p.R) v += O::ld(p.R, (int64_t)m * p.ldr + nc + e);
      O::st(p.C, (int64_t)m * p.ldc + nc + e, v);
    }
  });
}

// ---- split K over workgroups, with a workspace ------------------------------
//
// The same stream, cut differently: workgroup (split, panel) of the split
// kernel reads K slice `split` of a 256-column panel, its 4 waves taking 64
// columns each, so that together they read 512 contiguous bytes of every B
// row of the slice; with enough slices the grid holds several workgroups per
// compute unit.  Each wave writes its partial [M, 64] in fp32 to the
// workspace, ws[(split*M + m)*N + n]; a second kernel adds the partials of a
// cell in split order (deterministic, no atomics) and applies the epilogue.
struct SkinnySplit {
  static constexpr int WAVES = 4, THREADS = 64 * WAVES;
  static constexpr int PANEL = 64 * WAVES;    // columns per workgroup
  static constexpr int MIN_ITERS = 8;         // iterations of 32 k per slice at least
  static constexpr int TARGET_WGS = 512;      // two workgroups per compute unit
};

// The slices of a split run: `splits` slices of `per_split` iterations of 32
// k (the last one shorter), and the workspace they fill.  splits < 2: no
// split (the single-pass kernel is used).
struct SplitPlan {
  int splits, per_split;
  int64_t ws_bytes;
};
constexpr SplitPlan skinny_split_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t iters = (K + SkinnyTile::KW - 1) / SkinnyTile::KW;
  const int64_t panels = (N + SkinnySplit::PANEL - 1) / SkinnySplit::PANEL;
  int64_t splits = (SkinnySplit::TARGET_WGS + panels - 1) / panels;
  const int64_t most = iters / SkinnySplit::MIN_ITERS;
  splits = splits < most ? splits : most;
  if (splits < 2) return SplitPlan{1, (int)iters, 0};
  const int64_t per = (iters + splits - 1) / splits;
  splits = (iters + per - 1) / per;     // no empty slice
  return SplitPlan{(int)splits, (int)per, splits * M * N * 4};
}

template <int DT>
__global__ __launch_bounds__(SkinnySplit::THREADS) void gemm_skinny_split_kernel(
    GemmArgs p, float* ws, int splits, int per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int panels = (p.N + SkinnySplit::PANEL - 1) / SkinnySplit::PANEL;
  // consecutive workgroups take neighbouring panels of one slice
  const int split = blockIdx.x / panels, panel = blockIdx.x % panels;
  const int n0 = panel * SkinnySplit::PANEL + 64 * wave;
  if (n0 >= p.N) return;   // no barrier below: waves past N leave at once
  const int iters_total = (p.K + SkinnyTile::KW - 1) / SkinnyTile::KW;
  const int it0 = split * per_split;
  const int it1 = min(it0 + per_split, iters_total);
  f32x4 acc[4];
  skinny_stream<DT>(p, n0, it0, it1, lane, acc);
  // register r of acc[j]: row 4*(lane/16) + r, column n0 + 4*(lane%16) + j;
  // N % 4 == 0, so the lane's four columns are all inside or all outside
  const int n = n0 + 4 * (lane & 15);
  if (n >= p.N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * (lane >> 4) + r;
    if (m >= p.M) continue;
    *reinterpret_cast<f32x4*>(ws + ((int64_t)split * p.M + m) * p.N + n) =
        f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
  }
}

// Thread q of the reduction owns the run of four columns 4*(q % (N/4)) of
// row q / (N/4): the sum of the slices' partials in split order, then
// y = relu(sum * scale[m] + bias[n]) + R[m, n] (each term when present) and
// one rounding to the output type, as the single-pass kernel does.
template <int OT>
__global__ __launch_bounds__(256) void skinny_split_reduce_kernel(GemmArgs p, const float* ws,
                                                                  int splits) {
  using O = Out<OT>;
  const int64_t runs = p.N / 4;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)p.M * runs) return;
  const int m = (int)(q / runs), n = 4 * (int)(q % runs);
  f32x4 y = *reinterpret_cast<const f32x4*>(ws + (int64_t)m * p.N + n);
  for (int s = 1; s < splits; ++s) y += *reinterpret_cast<const f32x4*>(ws + ((int64_t)s * p.M + m) * p.N + n);
  float v[4] = {y[0], y[1], y[2], y[3]};
  const float sc = p.scale ? O::ld(p.scale, m) : 1.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (p.scale) v[e] *= sc;
    if (p.bias) v[e] += O::ld(p.bias, n + e);
    if (p.relu) v[e] = v[e] > 0.f ? v[e] : 0.f;
    if (p.R) v[e] += O::ld(p.R, (int64_t)m * p.ldr + n + e);
  }
  const int64_t c0 = (int64_t)m * p.ldc + n;
  if (p.epi_vec) {
    O::st4(p.C, c0, O::pack(v));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) O::st(p.C, c0 + e, v[e]);
  }
}

}  // namespace trt
