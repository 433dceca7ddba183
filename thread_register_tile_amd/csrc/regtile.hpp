// regtile.hpp -- register tiles of any logical shape, and the GEMM that runs
// them on general-purpose vector lanes.
//
// "My Triton From Scratch, Part 16: Register Tiles": a program instance owns
// a logical C tile of (lm, ln) results; a physical thread shape (tm, tn)
// cooperates on it, each thread holding a register tile of (lm/tm, ln/tn)
// accumulators.  Section "A strided ownership rule": thread (ti, tj),
// register (ri, rj) owns logical (ti + ri*tm, tj + rj*tn), which covers the
// tile exactly once whenever tm divides lm and tn divides ln -- so it needs
// no power-of-two sizes, unlike the GF(2) maps of the matrix-core tiles.
// Section "Choosing the physical thread shape": among divisor pairs (a of
// lm, b of ln) with a*b at most a thread budget, the largest by (a*b,
// min(a, b), b).  The pages' budget is one 32-thread warp; here it is at
// most one 64-lane wavefront.
//
// The kernel: one wavefront per logical tile.  Each K step of 16 stages the
// [lm x 16] A tile and the [16 x ln] B tile in LDS as fp32, row-major with
// an odd pitch of 17 floats, copied by all 64 lanes in the order in which
// each operand is contiguous in global memory.  Lanes t < tm*tn then read
// their lm/tm values of A and ln/tn values of B per k (immediate k offsets
// from row bases fixed for the whole kernel; the rows one read touches fall
// on distinct banks) and update every accumulator with one fp32 fused
// multiply-add.  When both tiles have at most 64 rows (at most kRegtilePF
// elements per lane), the global loads of step k+1 are issued into
// registers before step k's products and written to LDS after them, so
// their latency is hidden behind the arithmetic; larger tiles load each
// step's elements in batches of eight before its products.  The epilogue
// is the fused one of the matrix-core kernels, one element at a time.
// Registers per axis are bounded (kRegtileMaxRegs) so that every
// accumulator index is a compile-time constant; the kernel is instantiated
// for register bounds MRM x MRN in {1, 2, 4, 8} (with and without the
// prefetch), the launch taking the smallest bounds that hold (lm/tm,
// ln/tn).
#pragma once

#include <stdint.h>

#include "gemm_kernel.hpp"

namespace trt {

constexpr int kRegtileThreads = 64;   // one wavefront per tile
constexpr int kRegtileMaxRegs = 8;    // registers per axis
constexpr int kRegtileBK = 16;        // K step
constexpr int kRegtilePF = 16;        // prefetched elements per lane and operand (rows <= 64)
constexpr int kRegtilePitch = kRegtileBK + 1;   // LDS floats per tile row (odd: rows on distinct banks)

// The thread-shape policy: false if lm, ln or max_threads is not positive.
inline bool regtile_thread_shape(int64_t lm, int64_t ln, int64_t max_threads, int& tm, int& tn) {
  if (lm < 1 || ln < 1 || max_threads < 1) return false;
  int64_t best_p = 0, best_min = 0, best_b = 0;
  for (int64_t a = 1; a <= lm && a <= max_threads; ++a) {
    if (lm % a) continue;
    for (int64_t b = 1; b <= ln && a * b <= max_threads; ++b) {
      if (ln % b) continue;
      const int64_t p = a * b, mn = a < b ? a : b;
      if (p > best_p || (p == best_p && (mn > best_min || (mn == best_min && b > best_b)))) {
        best_p = p;
        best_min = mn;
        best_b = b;
        tm = (int)a;
        tn = (int)b;
      }
    }
  }
  return true;
}

// Strided ownership: thread t = ti*tn + tj, register r = ri*rn + rj.
__host__ __device__ __forceinline__ void regtile_coord(int t, int r, int tm, int tn, int rn,
                                                       int& row, int& col) {
  const int ti = t / tn, tj = t % tn, ri = r / rn, rj = r % rn;
  row = ti + ri * tm;
  col = tj + rj * tn;
}

struct RegtileArgs {
  GemmArgs g;
  int lm, ln, tm, tn, rm, rn;
  int opA, opB;
  int prefetch;   // the next K step's tiles are loaded during this one's products
};

template <int DT>
__device__ __forceinline__ float regtile_in(const void* X, int64_t i) {
  if constexpr (DT == DT_F32)
    return static_cast<const float*>(X)[i];
  else
    return to_f32<DT>(static_cast<const uint16_t*>(X)[i]);
}

template <int DT, int MRM, int MRN, bool PREFETCH>
__global__ __launch_bounds__(kRegtileThreads) void gemm_regtile_kernel(RegtileArgs p) {
  constexpr int BK = kRegtileBK;
  extern __shared__ float rt_lds[];
  const GemmArgs& g = p.g;
  const int lm = p.lm, ln = p.ln, tm = p.tm, tn = p.tn, rm = p.rm, rn = p.rn;
  constexpr int PITCH = kRegtilePitch;
  float* As = rt_lds;                // [lm][PITCH]: row r's k at r*PITCH + k
  float* Bs = rt_lds + lm * PITCH;   // [ln][PITCH]

  const int t = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / g.tiles_n) * lm, n0 = (tile % g.tiles_n) * ln;
  const bool active = t < tm * tn;
  const int ti = active ? t / tn : 0, tj = active ? t % tn : 0;

  float acc[MRM][MRN];
#pragma unroll
  for (int i = 0; i < MRM; ++i)
#pragma unroll
    for (int j = 0; j < MRN; ++j) acc[i][j] = 0.f;

  // Copy order: element e = t + 64*step of an operand tile is (row e/BK, k
  // e%BK) when k is contiguous in global memory, else (row e%rows, k
  // e/rows).  The second form steps each lane's (row, k) by the constant
  // (64 % rows, 64 / rows) with a carry instead of dividing per element.
  const int a_rows = p.opA ? lm : 0, b_rows = p.opB ? 0 : ln;   // 0: k contiguous
  const int a_r0 = a_rows ? t % a_rows : t / BK, a_k0 = a_rows ? t / a_rows : t % BK;
  const int a_dr = a_rows ? kRegtileThreads % a_rows : kRegtileThreads / BK;
  const int a_dk = a_rows ? kRegtileThreads / a_rows : 0;
  const int b_r0 = b_rows ? t % b_rows : t / BK, b_k0 = b_rows ? t / b_rows : t % BK;
  const int b_dr = b_rows ? kRegtileThreads % b_rows : kRegtileThreads / BK;
  const int b_dk = b_rows ? kRegtileThreads / b_rows : 0;

  // One operand tile: `rows` rows (m or n) x BK k, element (r, kk) read
  // from X[r*ld + k] (k contiguous) or X[k*ld + r], stored at S[r*PITCH + kk].
  // Eight elements per batch are loaded before any is written, so that
  // their global loads are in flight together.
  auto copy = [&](const void* X, int64_t ld, bool kc, int rows, int64_t r_base, int64_t r_lim,
                  int64_t k0, float* S, int r0, int kk0, int dr, int dk, bool carry) {
    int r = r0, kk = kk0;
    while (kk < BK && r < rows) {
      float v[8];
      int off[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in_tile = kk < BK && r < rows;
        const int64_t gr = r_base + r, k = k0 + kk;
        v[u] = 0.f;
        off[u] = in_tile ? r * PITCH + kk : -1;
        if (in_tile && gr < r_lim && k < g.K) v[u] = regtile_in<DT>(X, kc ? gr * ld + k : k * ld + gr);
        r += dr;
        kk += dk;
        if (carry && r >= rows) { r -= rows; ++kk; }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (off[u] >= 0) S[off[u]] = v[u];
    }
  };

  // The products of one K step from the staged tiles.  Register slots past
  // (rm, rn) read a valid element (the last row or column of the thread)
  // instead of branching, and feed accumulators the epilogue never stores;
  // a thread's rows start at offsets fixed for the whole kernel and k is
  // an immediate offset, so a K step's LDS reads need no address
  // arithmetic and can run ahead of its multiply-adds.
  int aoff[MRM], boff[MRN];
#pragma unroll
  for (int i = 0; i < MRM; ++i) aoff[i] = (ti + (i < rm ? i : rm - 1) * tm) * PITCH;
#pragma unroll
  for (int j = 0; j < MRN; ++j) boff[j] = (tj + (j < rn ? j : rn - 1) * tn) * PITCH;
  auto products = [&]() {
    if (!active) return;
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[MRM], b[MRN];
#pragma unroll
      for (int i = 0; i < MRM; ++i) a[i] = As[aoff[i] + kk];
#pragma unroll
      for (int j = 0; j < MRN; ++j) b[j] = Bs[boff[j] + kk];
#pragma unroll
      for (int i = 0; i < MRM; ++i)
#pragma unroll
        for (int j = 0; j < MRN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
  };

  if constexpr (PREFETCH) {
    // Lane t's elements e = t + 64u (u < PF) of an operand tile, in the
    // same order as the batched copy: k-contiguous storage gives (row
    // t/16 + 4u, k t%16), rows-contiguous storage (row e % rows, k
    // e / rows).  Their byte offsets from the K step's first element are
    // computed once (out of range where the row is outside the operand or
    // the element outside the tile); a buffer descriptor per K step, its
    // record count what is left of the operand, reads zero past the end.
    constexpr int PF = kRegtilePF;
    constexpr uint32_t NONE = 0x80000000u;
    const int64_t isz = DT == DT_F32 ? 4 : 2;
    auto offsets = [&](int64_t ld, bool kc, int rows, int64_t r_base, int64_t r_lim,
                       uint32_t (&off)[PF], int (&lo)[PF]) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int e = t + 64 * u;
        const int r = kc ? t / BK + 4 * u : e % rows, kk = kc ? t % BK : e / rows;
        const bool ok = r < rows && kk < BK && r_base + r < r_lim;
        off[u] = ok ? (uint32_t)((kc ? (r_base + r) * ld + kk : kk * ld + r_base + r) * isz) : NONE;
        lo[u] = r < rows && kk < BK ? r * PITCH + kk : -1;
      }
    };
    auto rsrc = [&](const void* X, int64_t bytes, int64_t adv) {
      int64_t left = bytes - adv;
      left = left < 0 ? 0 : left;
      return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)X + (adv < bytes ? adv : 0)),
                                               (short)0, (int)left, kBufferFormat);
    };
    auto fetch = [&](__amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[PF], bool zero, float (&v)[PF]) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if constexpr (DT == DT_F32)
          v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off[u], 0, 0));
        else
          v[u] = to_f32<DT>(__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(rs, off[u], 0, 0)));
        if (zero) v[u] = 0.f;
      }
    };
    // LDS: element (row, k) at row*PITCH + k; for k-contiguous storage
    // lane t's element u is (t/16 + 4u, t%16), a closed form
    // (one branch on the storage order per operand and step, not one per
    // element; an element outside the tile goes to the spare float after
    // both tiles instead of being masked, so no lane mask stays live)
    auto put = [&](float* S, bool kc, int rows, const float (&v)[PF], const int (&lo)[PF]) {
      const int off_spare = (int)(rt_lds + (lm + ln) * PITCH - S);  // the spare float
      if (kc) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int r = t / BK + 4 * u;
          S[r < rows ? r * PITCH + t % BK : off_spare] = v[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < PF; ++u) S[lo[u] >= 0 ? lo[u] : off_spare] = v[u];
      }
    };
    const bool akc = !p.opA, bkc = p.opB;
    uint32_t oa[PF], ob[PF];
    int la[PF], lb[PF];
    offsets(g.lda, akc, lm, m0, g.M, oa, la);
    offsets(g.ldb, bkc, ln, n0, g.N, ob, lb);
    float va[PF], vb[PF];
    // a k-contiguous element at k >= K lies inside the operand (the next
    // row); only the last K step has such elements, and only lanes whose k
    // t % 16 is past K
    // bytes per K step of each operand
    const int64_t a_step = BK * (akc ? 1 : g.lda) * isz, b_step = BK * (bkc ? 1 : g.ldb) * isz;
    auto step_loads = [&](int64_t k0) {
      const int64_t s = k0 / BK;
      const auto ra = rsrc(g.A, g.a_bytes, s * a_step), rb = rsrc(g.B, g.b_bytes, s * b_step);
      if (k0 + BK <= g.K) {   // (every step but a partial last one)
        fetch(ra, oa, false, va);
        fetch(rb, ob, false, vb);
      } else {
        const bool kout = k0 + t % BK >= g.K;
        fetch(ra, oa, akc && kout, va);
        fetch(rb, ob, bkc && kout, vb);
      }
    };
    step_loads(0);
    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
      put(As, akc, lm, va, la);
      put(Bs, bkc, ln, vb, lb);
      __syncthreads();
      if (k0 + BK < g.K) step_loads(k0 + BK);
      products();
      __syncthreads();
    }
  } else {
    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
      copy(g.A, g.lda, !p.opA, lm, m0, g.M, k0, As, a_r0, a_k0, a_dr, a_dk, a_rows != 0);
      copy(g.B, g.ldb, p.opB, ln, n0, g.N, k0, Bs, b_r0, b_k0, b_dr, b_dk, b_rows != 0);
      __syncthreads();
      products();
      __syncthreads();
    }
  }
  if (!active) return;

  // the fused epilogue, one owned element at a time:
  // y = relu(acc * scale[m] + bias[n]) + R[m][n], one rounding to the output type
  const OutAny O{g.out_dt};
#pragma unroll
  for (int i = 0; i < MRM; ++i) {
#pragma unroll
    for (int j = 0; j < MRN; ++j) {
      if (i >= rm || j >= rn) continue;
      const int64_t m = m0 + ti + i * tm, n = n0 + tj + j * tn;
      if (m >= g.M || n >= g.N) continue;
      float y = acc[i][j];
      if (g.scale) y *= O.ld(g.scale, m);
      if (g.bias) y += O.ld(g.bias, n);
      if (g.relu) y = y > 0.f ? y : 0.f;
      if (g.R) y += O.ld(g.R, m * g.ldr + n);
      O.st(g.C, m * g.ldc + n, y);
    }
  }
}

}  // namespace trt
