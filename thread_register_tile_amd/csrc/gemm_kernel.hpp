// gemm_kernel.hpp -- the register-tile GEMM kernel for gfx950 (CDNA4).
//
// One workgroup owns one logical [BM, BN] tile of C.  Per K step it moves the
// [BM, BK] tile of A and the [BK, BN] tile of B cooperatively from global
// memory into LDS (double-buffered: the next step's loads are in flight while
// the current step computes), each wave reads its matrix-core fragments from
// LDS and accumulates its register tile in fp32, and after the last step the
// fused epilogue adds bias, applies ReLU, adds the residual, rounds once and
// stores with per-register masks.
//
// Page correspondence:
//   * the GEMM arrangement, fp32 accumulator and single final cast -- NineToothed
//     "Named layouts", GEMM arrangement and section "Contract";
//   * cooperative copies -- "My Triton From Scratch, Part 12: CUDA Tile
//     Layouts", section "Cooperative tile layouts";
//   * several accumulators per thread, loop-carried across K steps, masked
//     per register, broadcast bias storage -- "My Triton From Scratch, Part
//     16: Register Tiles", sections "Computing several dot results",
//     "Broadcasts cannot be treated as full register tiles", "Masks and
//     stores", "Register-valued loop-carried accumulators";
//   * swizzled shared tiles, vector loads, double buffering, 16-bit inputs on
//     matrix cores -- the items that page's "What Version 16 does not
//     optimize" leaves open.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace trt {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element types: inputs are DT_F16 or DT_BF16; the output (and the epilogue
// operands, stored in the output type) may also be DT_F32.
enum : int { DT_F16 = 1, DT_BF16 = 2, DT_F32 = 3 };

// ---- element conversions ----------------------------------------------------

template <int DT>
__device__ __forceinline__ float to_f32(uint32_t h16);
template <>
__device__ __forceinline__ float to_f32<DT_F16>(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}
template <>
__device__ __forceinline__ float to_f32<DT_BF16>(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Round to nearest, ties to even (the hardware conversions' default mode).
template <int DT>
__device__ __forceinline__ uint32_t from_f32(float x);
template <>
__device__ __forceinline__ uint32_t from_f32<DT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <>
__device__ __forceinline__ uint32_t from_f32<DT_BF16>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two values rounded as from_f32 rounds them, packed with the first in the
// low half (one conversion instruction on gfx950 for both types).
template <int DT>
__device__ __forceinline__ uint32_t pack2_f32(float lo, float hi) {
  if constexpr (DT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// ---- matrix core ---------------------------------------------------------------

// Instruction classes of __builtin_amdgcn_sched_group_barrier masks.
enum : int {
  SG_VALU = 0x002,
  SG_MFMA = 0x008,
  SG_DS_READ = 0x100,
  SG_DS_WRITE = 0x200,
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<DT_F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<DT_BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<DT_F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<DT_BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- output elements ---------------------------------------------------------------

// Cache-policy operand of the buffer load / store builtins: non-temporal.
constexpr int kNonTemporal = 2;
// Format word (word 3) of the buffer descriptors this library builds.
constexpr int kBufferFormat = 0x00020000;
// C, bias, residual and row scale hold elements of the output type OT.  Out
// reads and writes one element, or a run of four consecutive ones as one
// vector (8 bytes for 16-bit types, 16 for binary32) when the caller has
// checked that the run is in range and aligned.
template <int OT>
struct Out {
  using Vec = u32x2;
  static constexpr int BYTES = 2;
  __device__ static float ld(const void* p, int64_t i) {
    return to_f32<OT>(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static void st(void* p, int64_t i, float y) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)from_f32<OT>(y);
  }
  __device__ static Vec ld4(const void* p, int64_t i) {
    return *reinterpret_cast<const Vec*>(static_cast<const uint16_t*>(p) + i);
  }
  __device__ static void st4(void* p, int64_t i, Vec v) {
    *reinterpret_cast<Vec*>(static_cast<uint16_t*>(p) + i) = v;
  }
  __device__ static float elem(Vec v, int e) {
    return to_f32<OT>((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xFFFFu));
  }
  __device__ static Vec pack(const float (&y)[4]) {
    return Vec{pack2_f32<OT>(y[0], y[1]), pack2_f32<OT>(y[2], y[3])};
  }
  // a run of four through a buffer descriptor at byte offset off, read or
  // written once (non-temporal: the residual and C of the fast epilogue); a
  // load past the record count reads zero, a store past it is dropped
  __device__ static Vec ld4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, kNonTemporal);
  }
  __device__ static void st4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, Vec v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)off, 0, kNonTemporal);
  }
  __device__ static float ld_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return to_f32<OT>(__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0));
  }
};
template <>
struct Out<DT_F32> {
  using Vec = f32x4;
  static constexpr int BYTES = 4;
  __device__ static float ld(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void st(void* p, int64_t i, float y) { static_cast<float*>(p)[i] = y; }
  __device__ static Vec ld4(const void* p, int64_t i) {
    return *reinterpret_cast<const Vec*>(static_cast<const float*>(p) + i);
  }
  __device__ static void st4(void* p, int64_t i, Vec v) {
    *reinterpret_cast<Vec*>(static_cast<float*>(p) + i) = v;
  }
  __device__ static float elem(Vec v, int e) { return v[e]; }
  __device__ static Vec pack(const float (&y)[4]) { return Vec{y[0], y[1], y[2], y[3]}; }
  __device__ static Vec ld4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(Vec, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, kNonTemporal));
  }
  __device__ static void st4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, Vec v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)off, 0, kNonTemporal);
  }
  __device__ static float ld_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
  }
};

// Calls f.template operator()<OT>() for the run-time output type (uniform
// over the grid, so the branch costs one scalar compare).
template <class F>
__device__ __forceinline__ void with_out_type(int out_dt, F&& f) {
  if (out_dt == DT_F16)
    f.template operator()<DT_F16>();
  else if (out_dt == DT_BF16)
    f.template operator()<DT_BF16>();
  else
    f.template operator()<DT_F32>();
}

// ---- kernel arguments --------------------------------------------------------------

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;               // output, elements of out_dt
  const void* bias;      // [N] of out_dt, or null
  const void* R;         // residual of out_dt, R(m,n) = R[m*ldr + n], or null
  const void* scale;     // row scale [M] of out_dt, or null
  int64_t lda, ldb, ldc, ldr;
  int32_t M, N, K;
  int32_t relu;
  int32_t out_dt;        // DT_F16, DT_BF16 or DT_F32
  int32_t epi_vec;       // 4-element vector epilogue allowed (alignment holds)
  int32_t tiles_m, tiles_n;
  int64_t a_bytes, b_bytes;  // byte extents of the A and B operands
};

// Workgroup id -> (tile row, tile column).  Consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, each with its own L2: first give
// every XCD a contiguous range of tile ids, then walk tiles in groups of
// GROUP_M tile rows, column by column, so the tiles an XCD runs together
// share A row panels and B column panels in its L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int x = bid & 7, local = bid >> 3;
  const int q = total >> 3, rem = total & 7;
  const int id = x * q + (x < rem ? x : rem) + local;
  const int per_group = GROUP_M * tiles_n;
  const int grp = id / per_group;
  const int first = grp * GROUP_M;
  const int rows = (tiles_m - first) < GROUP_M ? (tiles_m - first) : GROUP_M;
  const int in = id - grp * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

// ---- global -> registers ---------------------------------------------------------

// 8 consecutive 16-bit elements starting at src, n of them valid (the rest
// read as zero).  VEC: src is 16-byte aligned whenever n == 8.
template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t* src, int n) {
  if (VEC && n >= 8) return *reinterpret_cast<const u32x4*>(src);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (e < n) ? (uint32_t)src[e] : 0u;
  return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
               h[6] | (h[7] << 16)};
}

// Operand stored with k contiguous: element (r, k) at X[(row0 + r)*ld + k].
template <class TL, int R, bool VEC>
struct KContigOperand {
  using Map = typename TL::template KContig<R>;
  static constexpr int ITERS = Map::ITERS;
  u32x4 st[ITERS];

  template <bool CHECK>
  __device__ __forceinline__ void load(const uint16_t* X, int64_t ld, int row0, int rows,
                                       int k0, int K, int t) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      if (Map::ITEMS % TL::THREADS != 0 && !Map::active(t, i)) continue;
      const int r = row0 + Map::row(t, i);
      const int k = k0 + 8 * Map::g(t, i);
      const uint16_t* src = X + (int64_t)r * ld + k;
      if (!CHECK) {
        st[i] = load8<VEC>(src, 8);
      } else {
        int n = K - k;
        n = n < 0 ? 0 : (n > 8 ? 8 : n);
        if (r >= rows) n = 0;
        st[i] = load8<VEC>(src, n);
      }
    }
  }

  __device__ __forceinline__ void store(u32x4* lds, int t) const {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      if (Map::ITEMS % TL::THREADS != 0 && !Map::active(t, i)) continue;
      lds[TL::lds_slot(Map::row(t, i), Map::g(t, i))] = st[i];
    }
  }
};

// Operand stored with its rows (m for A^T, n for B) contiguous: element
// (r, k) at X[k*ld + row0 + r].  Each item is an 8x8 block: eight 16-byte
// runs along r on consecutive k, transposed in registers into eight k-runs.
template <class TL, int R, bool VEC>
struct MNContigOperand {
  using Map = typename TL::template MNContig<R>;
  static constexpr int ITERS = Map::ITERS;
  u32x4 st[ITERS][8];

  template <bool CHECK>
  __device__ __forceinline__ void load(const uint16_t* X, int64_t ld, int row0, int rows,
                                       int k0, int K, int t) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      if (Map::ITEMS % TL::THREADS != 0 && !Map::active(t, i)) continue;
      const int r = row0 + 8 * Map::rb(t, i);
      const int kb = k0 + 8 * Map::g(t, i);
      int nr = rows - r;
      nr = nr < 0 ? 0 : (nr > 8 ? 8 : nr);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint16_t* src = X + (int64_t)(kb + j) * ld + r;
        if (!CHECK)
          st[i][j] = load8<VEC>(src, 8);
        else
          st[i][j] = load8<VEC>(src, (kb + j < K) ? nr : 0);
      }
    }
  }

  __device__ __forceinline__ void store(u32x4* lds, int t) const {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      if (Map::ITEMS % TL::THREADS != 0 && !Map::active(t, i)) continue;
      const int rb = Map::rb(t, i), g = Map::g(t, i);
      // st[i][j] holds (r = 8rb + e, k = 8g + j) for e = 0..7, two per word:
      // word q has e = 2q (low half) and e = 2q + 1 (high half).  Output row
      // e gathers k = 0..7, two per word: word p has k = 2p, 2p + 1.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 lo, hi;  // rows e = 2q and e = 2q + 1
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a = st[i][2 * p][q], b = st[i][2 * p + 1][q];
          lo[p] = (a & 0xFFFFu) | (b << 16);
          hi[p] = (a >> 16) | (b & 0xFFFF0000u);
        }
        lds[TL::lds_slot(8 * rb + 2 * q, g)] = lo;
        lds[TL::lds_slot(8 * rb + 2 * q + 1, g)] = hi;
      }
    }
  }
};

template <class TL, int R, bool KC, bool VEC>
using Operand = typename std::conditional<KC, KContigOperand<TL, R, VEC>,
                                          MNContigOperand<TL, R, VEC>>::type;

// ---- fused epilogue --------------------------------------------------------------
// The output type of the generic kernels' epilogue is read at run time: one
// copy of the (fully unrolled) epilogue serves all three output types, each
// element access branching on the uniform type code.
struct OutAny {
  int dt;
  __device__ __forceinline__ float cvt16(uint32_t h) const {
    return dt == DT_BF16 ? to_f32<DT_BF16>(h) : to_f32<DT_F16>(h);
  }
  __device__ __forceinline__ uint32_t rnd16(float y) const {
    return dt == DT_BF16 ? from_f32<DT_BF16>(y) : from_f32<DT_F16>(y);
  }
  __device__ __forceinline__ float ld(const void* p, int64_t i) const {
    if (dt == DT_F32) return static_cast<const float*>(p)[i];
    return cvt16(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ __forceinline__ void st(void* p, int64_t i, float y) const {
    if (dt == DT_F32)
      static_cast<float*>(p)[i] = y;
    else
      static_cast<uint16_t*>(p)[i] = (uint16_t)rnd16(y);
  }
  // four consecutive elements from i (aligned, in range)
  __device__ __forceinline__ void ld4(const void* p, int64_t i, float (&v)[4]) const {
    if (dt == DT_F32) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
      v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
      v[0] = cvt16(w[0] & 0xFFFFu); v[1] = cvt16(w[0] >> 16);
      v[2] = cvt16(w[1] & 0xFFFFu); v[3] = cvt16(w[1] >> 16);
    }
  }
  __device__ __forceinline__ void st4(void* p, int64_t i, const float (&y)[4]) const {
    if (dt == DT_F32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = f32x4{y[0], y[1], y[2], y[3]};
    } else {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p) + i) =
          u32x2{rnd16(y[0]) | (rnd16(y[1]) << 16), rnd16(y[2]) | (rnd16(y[3]) << 16)};
    }
  }
};

// Per accumulator register ("My Triton From Scratch, Part 16: Register Tiles",
// sections "Pointer tiles" and "Masks and stores"): the register's (row, col)
// comes from the tile's ownership map, the bias is read once per owned column
// (it is broadcast along m) and the row scale once per owned row (broadcast
// along n), y = relu(acc * scale + bias) + R is evaluated in fp32, rounded
// once to the output type, and stored under its own mask.  A lane owns four
// consecutive columns of a row per fragment, stored as one vector when the
// whole run is in range and the buffers are aligned.
template <class TL, class AccT>
__device__ __forceinline__ void epilogue_store(const GemmArgs& p,
                                               const AccT (&acc)[TL::FM][TL::FN], int m0,
                                               int n0, int lane, int wave) {
  const OutAny O{p.out_dt};
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
#pragma unroll
      for (int q = 0; q < TL::FRAG_REGS / 4; ++q) {
        const int reg = TL::FRAG_REGS * (i * TL::FN + j) + 4 * q;
        const int m = m0 + TL::owner_row(reg, lane, wave);
        const int n = n0 + TL::owner_col(reg, lane, wave);  // this run: n..n+3
        if (m >= p.M) continue;
        float y[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        const bool vec = p.epi_vec && (n + 4 <= p.N);
        if (p.scale) {
          const float s = O.ld(p.scale, m);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] *= s;
        }
        if (p.bias) {
          if (vec) {
            float bb[4];
            O.ld4(p.bias, n, bb);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] += bb[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) y[e] += O.ld(p.bias, n + e);
          }
        }
        if (p.relu) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = y[e] > 0.f ? y[e] : 0.f;
        }
        if (p.R) {
          const int64_t r0 = (int64_t)m * p.ldr + n;
          if (vec) {
            float rr[4];
            O.ld4(p.R, r0, rr);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] += rr[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) y[e] += O.ld(p.R, r0 + e);
          }
        }
        const int64_t c0 = (int64_t)m * p.ldc + n;
        if (vec) {
          O.st4(p.C, c0, y);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) O.st(p.C, c0 + e, y[e]);
        }
      }
    }
  }
}

// ---- the kernel -------------------------------------------------------------------

// A_KC: A stored with k contiguous (op N); otherwise A^T (op T).
// B_KC: B stored with k contiguous (B^T, op T); otherwise row-major (op N).
// VEC:  16-byte aligned operand rows, so chunks load as one vector.
template <class TL, int DT, bool A_KC, bool B_KC, bool VEC>
__global__ __launch_bounds__(TL::THREADS) void gemm_kernel(GemmArgs p) {
  static_assert(TL::MF == 16, "the generic kernel runs 16x16x32 fragments");
  constexpr int G = TL::G;
  __shared__ u32x4 lds[2][(TL::BM + TL::BN) * G];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int tm, tn;
  tile_of<8>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * TL::BM, n0 = tn * TL::BN;
  const bool full_mn = (m0 + TL::BM <= p.M) && (n0 + TL::BN <= p.N);

  Operand<TL, TL::BM, A_KC, VEC> a;
  Operand<TL, TL::BN, B_KC, VEC> b;

  f32x4 acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (p.K + TL::BK - 1) / TL::BK;

  auto load_step = [&](int kt) {
    const int k0 = kt * TL::BK;
    if (full_mn && k0 + TL::BK <= p.K) {
      a.template load<false>(p.A, p.lda, m0, p.M, k0, p.K, t);
      b.template load<false>(p.B, p.ldb, n0, p.N, k0, p.K, t);
    } else {
      a.template load<true>(p.A, p.lda, m0, p.M, k0, p.K, t);
      b.template load<true>(p.B, p.ldb, n0, p.N, k0, p.K, t);
    }
  };

  // wave position in the workgroup tile (thread shape WM x WN)
  const int wrow = (wave / TL::WN) * TL::WTM;
  const int wcol = (wave % TL::WN) * TL::WTN;

  load_step(0);
  a.store(lds[0], t);
  b.store(lds[0] + TL::BM * G, t);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_step(kt + 1);

    const u32x4* la = lds[cur];
    const u32x4* lb = lds[cur] + TL::BM * G;
#pragma unroll
    for (int ks = 0; ks < TL::KSUB; ++ks) {
      const int g = 4 * ks + (lane >> 4);
      u32x4 af[TL::FM], bf[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) af[i] = la[TL::lds_slot(wrow + 16 * i + (lane & 15), g)];
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) bf[j] = lb[TL::lds_slot(wcol + 16 * j + (lane & 15), g)];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = mfma16<DT>(bf[j], af[i], acc[i][j]);
    }

    if (kt + 1 < nk) {
      a.store(lds[cur ^ 1], t);
      b.store(lds[cur ^ 1] + TL::BM * G, t);
    }
    __syncthreads();
  }

  epilogue_store<TL>(p, acc, m0, n0, lane, wave);
}

}  // namespace trt
