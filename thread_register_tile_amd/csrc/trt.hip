// trt.hip -- the C ABI of libtrt.so: validation, tile selection, launches,
// layout introspection and the matrix-core probe.  Declarations and the
// contract of every entry point are in include/trt.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/trt.h"
#include "gemm_kernel.hpp"
#include "gemm_skinny.hpp"
#include "launch.hpp"
#include "reduce.hpp"
#include "regtile.hpp"
#include "tiles.hpp"
#include "validate.hpp"

namespace {

thread_local std::string g_err;

trt_status fail(trt_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// The status of one launch, as the runtime returned it for that launch.
trt_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(TRT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  g_err.clear();
  return TRT_OK;
}

using trt::GemmArgs;

// ---- compiled tiles ------------------------------------------------------------

using trt::Tile256;
using trt::Tile256x192D;
using trt::Tile256D;
using trt::Tile64;
using trt::Tile128;
using trt::Tile128D;
using trt::TileTiny;

// Whether the pipelined direct-to-LDS kernel applies: aligned 16-byte operand
// rows; every 16-byte copy wholly inside or wholly outside its operand's
// extent (the buffer record check drops a copy that straddles the end as a
// whole), i.e. K % 8 == 0 for a k-contiguous operand and M (N) % 8 == 0 for
// a rows-contiguous A (B); rows of a rows-contiguous operand that do not
// overlap (lda >= M, ldb >= N), so that its rows k >= K on a partial last K
// step start past the extent and read as zero; operand extents addressable
// by 32-bit offsets.  Other shapes and strides take the generic kernel,
// which masks k >= K explicitly.
bool dma_ok(const GemmArgs& a, int opA, int opB, bool vec) {
  const bool a_kc = opA == TRT_OP_N, b_kc = opB == TRT_OP_T;
  // every copy's byte offset from its K step's first byte, plus the
  // descriptor bias of up to 3 KiB, stays below 2^31: k-contiguous, the
  // operand's rows padded to a 256-row tile; rows-contiguous, 32 k rows
  // plus a padded row
  constexpr int64_t LIM = (int64_t(1) << 31) - 4096;
  auto pad = [](int64_t n) { return (n + 255) / 256 * 256; };
  auto fits = [&](bool kc, int64_t rows, int64_t ld, int64_t bytes) {
    const int64_t span = kc ? pad(rows) * ld * 2 : 32 * ld * 2 + pad(rows) * 2;
    return bytes < LIM && span < LIM;
  };
  return vec && (a_kc ? a.K % 8 == 0 : a.M % 8 == 0 && a.lda >= a.M) &&
         (b_kc ? a.K % 8 == 0 : a.N % 8 == 0 && a.ldb >= a.N) &&
         fits(a_kc, a.M, a.lda, a.a_bytes) && fits(b_kc, a.N, a.ldb, a.b_bytes);
}

// Whether the streaming kernel applies (M <= 16, A k-contiguous, B
// row-major, aligned vector rows, whole vector runs at the K and N edges).
bool skinny_ok(const GemmArgs& a, int opA, int opB) {
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; };
  return a.M <= 16 && opA == TRT_OP_N && opB == TRT_OP_N && al(a.A, 16) && a.lda % 8 == 0 &&
         al(a.B, 8) && a.ldb % 4 == 0 && a.K % 8 == 0 && a.N % 4 == 0;
}

// The streaming tile: the skinny kernel when it applies, otherwise the
// generic kernel on the 16x64 tile.
hipError_t launch_tile_skinny(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s) {
  if (!skinny_ok(a, opA, opB)) return trt::launch_generic<TileTiny>(a, dt, opA, opB, vec, s);
  return trt::launch_skinny(a, dt, s);
}

template <class TL>
hipError_t launch_tile(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s) {
  return trt::launch_generic<TL>(a, dt, opA, opB, vec, s);
}

// The pipelined tile: the direct-to-LDS kernel when it applies, otherwise the
// generic kernel on a tile of the same width (with 16x16 fragments).
template <class TL>
hipError_t launch_tile_dma(GemmArgs a, int dt, int opA, int opB, bool vec, hipStream_t s) {
  if (!dma_ok(a, opA, opB, vec)) {
    if constexpr (TL::BM == 128) return trt::launch_generic<trt::Tile128>(a, dt, opA, opB, vec, s);
    else return trt::launch_generic<trt::Tile256F>(a, dt, opA, opB, vec, s);
  }
  return trt::launch_pipelined<TL>(a, dt, opA, opB, s);
}

// ---- layout maps (host and device evaluate the same functions) ---------------

template <class TL, class = void>
struct HasCopyMaps : std::false_type {};
template <class TL>
struct HasCopyMaps<TL, std::void_t<decltype(TL::COPY_MAPS)>> : std::true_type {};

template <class TL>
TRT_HD int64_t map_size(int map) {
  if constexpr (!HasCopyMaps<TL>::value) {
    return map == TRT_MAP_C_OWNER ? (int64_t)TL::WAVES * 64 * TL::REGS : -1;
  } else if constexpr (!TL::POW2) {
    // (BK == 32 for every such tile)
    // a tile of the pipelined kernel only: its ownership and slot maps
    switch (map) {
      case TRT_MAP_C_OWNER: return (int64_t)TL::WAVES * 64 * TL::REGS;
      case TRT_MAP_DMA_KC_SLOT_A: return (int64_t)TL::BM * 4;
      case TRT_MAP_DMA_KC_SLOT_B: return (int64_t)TL::BN * 4;
      case TRT_MAP_DMA_MN_SLOT_A: return (int64_t)32 * (TL::BM / 8);
      case TRT_MAP_DMA_MN_SLOT_B: return (int64_t)32 * (TL::BN / 8);
      default: return -1;
    }
  } else {
  constexpr bool dma = TL::BK == 32;
  using KA = typename TL::template KContig<TL::BM>;
  using MA = typename TL::template MNContig<TL::BM>;
  using KB = typename TL::template KContig<TL::BN>;
  using MB = typename TL::template MNContig<TL::BN>;
  switch (map) {
    case TRT_MAP_C_OWNER: return (int64_t)TL::WAVES * 64 * TL::REGS;
    case TRT_MAP_LDS_SLOT_A: return (int64_t)TL::BM * TL::G;
    case TRT_MAP_LDS_SLOT_B: return (int64_t)TL::BN * TL::G;
    case TRT_MAP_COPY_KCONTIG_A: return (int64_t)KA::ITERS * TL::THREADS;
    case TRT_MAP_COPY_MNCONTIG_A: return (int64_t)MA::ITERS * TL::THREADS;
    case TRT_MAP_COPY_KCONTIG_B: return (int64_t)KB::ITERS * TL::THREADS;
    case TRT_MAP_COPY_MNCONTIG_B: return (int64_t)MB::ITERS * TL::THREADS;
    case TRT_MAP_DMA_KC_SLOT_A: return dma ? (int64_t)TL::BM * 4 : -1;
    case TRT_MAP_DMA_KC_SLOT_B: return dma ? (int64_t)TL::BN * 4 : -1;
    case TRT_MAP_DMA_MN_SLOT_A: return dma && TL::BM >= 128 ? (int64_t)32 * (TL::BM / 8) : -1;
    case TRT_MAP_DMA_MN_SLOT_B: return dma && TL::BN >= 128 ? (int64_t)32 * (TL::BN / 8) : -1;
    default: return -1;
  }
  }
}

template <class TL, class Map>
TRT_HD void eval_kcontig(int64_t x, int& r, int& c) {
  const int t = (int)(x % TL::THREADS), i = (int)(x / TL::THREADS);
  if (Map::active(t, i)) { r = Map::row(t, i); c = Map::g(t, i); }
  else { r = -1; c = -1; }
}

template <class TL, class Map>
TRT_HD void eval_mncontig(int64_t x, int& r, int& c) {
  const int t = (int)(x % TL::THREADS), i = (int)(x / TL::THREADS);
  if (Map::active(t, i)) { r = Map::rb(t, i); c = Map::g(t, i); }
  else { r = -1; c = -1; }
}

template <class TL>
TRT_HD void eval_map(int map, int64_t x, int& r, int& c) {
  if constexpr (!HasCopyMaps<TL>::value) {
    const int reg = (int)(x % TL::REGS);
    const int lane = (int)((x / TL::REGS) % 64);
    const int wave = (int)(x / (TL::REGS * 64));
    r = map == TRT_MAP_C_OWNER ? TL::owner_row(reg, lane, wave) : -1;
    c = map == TRT_MAP_C_OWNER ? TL::owner_col(reg, lane, wave) : -1;
    return;
  } else {
  switch (map) {
    case TRT_MAP_C_OWNER: {
      const int reg = (int)(x % TL::REGS);
      const int lane = (int)((x / TL::REGS) % 64);
      const int wave = (int)(x / (TL::REGS * 64));
      r = TL::owner_row(reg, lane, wave);
      c = TL::owner_col(reg, lane, wave);
      return;
    }
    case TRT_MAP_LDS_SLOT_A:
    case TRT_MAP_LDS_SLOT_B:
      r = TL::lds_slot((int)(x / TL::G), (int)(x % TL::G));
      c = 0;
      return;
    case TRT_MAP_COPY_KCONTIG_A:
      if constexpr (TL::POW2) eval_kcontig<TL, typename TL::template KContig<TL::BM>>(x, r, c);
      return;
    case TRT_MAP_COPY_MNCONTIG_A:
      if constexpr (TL::POW2) eval_mncontig<TL, typename TL::template MNContig<TL::BM>>(x, r, c);
      return;
    case TRT_MAP_COPY_KCONTIG_B:
      if constexpr (TL::POW2) eval_kcontig<TL, typename TL::template KContig<TL::BN>>(x, r, c);
      return;
    case TRT_MAP_COPY_MNCONTIG_B:
      if constexpr (TL::POW2) eval_mncontig<TL, typename TL::template MNContig<TL::BN>>(x, r, c);
      return;
    case TRT_MAP_DMA_KC_SLOT_A:
    case TRT_MAP_DMA_KC_SLOT_B:
      r = TL::kc_slot((int)(x / 4), (int)(x % 4));
      c = 0;
      return;
    case TRT_MAP_DMA_MN_SLOT_A:
      r = TL::template mn_slot<TL::BM>((int)(x / (TL::BM / 8)), (int)(x % (TL::BM / 8)));
      c = 0;
      return;
    case TRT_MAP_DMA_MN_SLOT_B:
      r = TL::template mn_slot<TL::BN>((int)(x / (TL::BN / 8)), (int)(x % (TL::BN / 8)));
      c = 0;
      return;
    default: r = c = -1; return;
  }
  }
}

template <class TL>
__global__ void dump_kernel(int map, int32_t* rows, int32_t* cols, int64_t n) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= n) return;
  int r, c;
  eval_map<TL>(map, x, r, c);
  rows[x] = r;
  cols[x] = c;
}

template <int DT>
__global__ __launch_bounds__(64) void probe_kernel(const trt::u32x4* a, const trt::u32x4* b,
                                                    trt::f32x4* c) {
  const int l = threadIdx.x;
  c[l] = trt::mfma16<DT>(a[l], b[l], trt::f32x4{0.f, 0.f, 0.f, 0.f});
}

template <int DT>
__global__ __launch_bounds__(64) void probe32_kernel(const trt::u32x4* a, const trt::u32x4* b,
                                                      trt::f32x16* c) {
  const int l = threadIdx.x;
  c[l] = trt::mfma32<DT>(a[l], b[l], trt::f32x16{});
}

// ---- tile registry ---------------------------------------------------------------

struct TileEntry {
  int bm, bn, bk, wm, wn, regs, frag;
  hipError_t (*launch)(GemmArgs, int, int, int, bool, hipStream_t);
  int64_t (*size)(int);
  void (*eval)(int, int64_t, int&, int&);
  hipError_t (*dump)(int, int32_t*, int32_t*, int64_t, hipStream_t);
  int rank, in_bits, out_bits;
};

template <class TL>
hipError_t dump_launch(int map, int32_t* rows, int32_t* cols, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  return trt::launch(dump_kernel<TL>, dim3((unsigned)blocks), dim3(256), 0, s, map, rows, cols, n);
}

template <class TL>
int64_t size_host(int map) { return map_size<TL>(map); }

template <class TL>
void eval_host(int map, int64_t x, int& r, int& c) { eval_map<TL>(map, x, r, c); }

template <class TL, bool DMA>
constexpr auto launcher() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return &launch_tile_skinny;
  else if constexpr (DMA) return &launch_tile_dma<TL>;
  else return &launch_tile<TL>;
}

template <class TL>
constexpr int tile_bk() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return TL::KW * TL::WAVES;
  else return TL::BK;
}
template <class TL>
constexpr int tile_wm() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return TL::WAVES;
  else return TL::WM;
}
template <class TL>
constexpr int tile_wn() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return 1;
  else return TL::WN;
}
template <class TL>
constexpr int tile_mf() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return 16;
  else return TL::MF;
}

template <class TL>
constexpr bool tile_is_gf2() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return true;
  else return TL::POW2;
}

template <class TL>
constexpr bool ownership_checked() {
  if constexpr (std::is_same_v<TL, trt::SkinnyTile>) return TL::owner_matches_bases();
  else if constexpr (TL::POW2) return TL::owner_matches_bases();
  else return TL::owner_exactly_once();
}

template <class TL, bool DMA = false>
constexpr TileEntry entry() {
  // power-of-two tiles: the kernel's ownership arithmetic equals its GF(2)
  // bases (whose full rank is asserted in layout.hpp); other tiles: every
  // element owned exactly once, by enumeration
  static_assert(ownership_checked<TL>(), "kernel ownership: exactly once");
  if constexpr (tile_is_gf2<TL>())
    return TileEntry{TL::BM, TL::BN, tile_bk<TL>(), tile_wm<TL>(), tile_wn<TL>(), TL::REGS,
                     tile_mf<TL>(), launcher<TL, DMA>(), &size_host<TL>, &eval_host<TL>,
                     &dump_launch<TL>, TL::c_map().rank(), TL::C_IN_BITS,
                     trt::ilog2(TL::BM * TL::BN)};
  else
    return TileEntry{TL::BM, TL::BN, tile_bk<TL>(), tile_wm<TL>(), tile_wn<TL>(), TL::REGS,
                     tile_mf<TL>(), launcher<TL, DMA>(), &size_host<TL>, &eval_host<TL>,
                     &dump_launch<TL>, -1, -1, -1};
}

const TileEntry kTiles[] = {entry<TileTiny>(), entry<Tile64>(), entry<Tile128>(),
                            entry<Tile256>(), entry<Tile256D, true>(),
                            entry<Tile256x192D, true>(), entry<Tile128D, true>(),
                            entry<trt::SkinnyTile>()};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

const TileEntry* find_tile(const trt_tile* t) {
  for (const TileEntry& e : kTiles)
    if (e.bm == t->bm && e.bn == t->bn && e.bk == t->bk) return &e;
  return nullptr;
}

const TileEntry* tile_named(int bm, int bn, int bk) {
  const trt_tile t{bm, bn, bk};
  return find_tile(&t);
}

// Tile choice when the caller names none.  M <= 16: the streaming tile.
// Otherwise, when either 256-wide pipelined tile gives the 256 compute units
// a full wave of workgroups, the one that needs the least work per compute
// unit: rounds of 256 workgroups times the tile's area (the 256x192 tile
// fills all compute units where 256x256 tiles would leave some idle).
// Smaller problems take the pipelined 128x128 tile (two workgroups per
// compute unit) when it gives at least 64 workgroups, else the generic
// kernel on 64x64 tiles.
const TileEntry* choose_tile(int64_t M, int64_t N) {
  auto count = [&](const TileEntry* e) { return ((M + e->bm - 1) / e->bm) * ((N + e->bn - 1) / e->bn); };
  auto cost = [&](const TileEntry* e) { return (count(e) + 255) / 256 * e->bm * e->bn; };
  if (M <= 16) return tile_named(16, 64, 256);
  const TileEntry* big = tile_named(256, 256, 32);
  const TileEntry* wide = tile_named(256, 192, 32);
  if (count(big) >= 192 || count(wide) >= 192) return cost(wide) < cost(big) ? wide : big;
  if (count(tile_named(128, 128, 32)) >= 64) return tile_named(128, 128, 32);
  return tile_named(64, 64, 64);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

// Plain streaming read of x (n 16-byte words): every wave reads runs of 128
// consecutive words (2 KiB, two non-temporal loads per lane) in turn, the
// runs dealt round-robin over all waves of the grid, and XORs what it read;
// each workgroup writes one 16-byte digest, so the XOR of all digests is the
// XOR of all words.  A memory-bound yardstick for the streaming kernels.
constexpr int kReadProbeBlocks = 2048;
__global__ __launch_bounds__(256) void hbm_read_kernel(const trt::u32x4* __restrict__ x, int64_t n,
                                                       trt::u32x4* sink) {
  __shared__ trt::u32x4 part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t runs = n / 128;
  trt::u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < runs; r += (int64_t)gridDim.x * 4) {
    const trt::u32x4 v0 = __builtin_nontemporal_load(&x[128 * r + lane]);
    const trt::u32x4 v1 = __builtin_nontemporal_load(&x[128 * r + 64 + lane]);
    acc ^= v0 ^ v1;
  }
  // the words after the last whole run, one per thread of the grid
  for (int64_t i = 128 * runs + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    acc ^= x[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] ^= __shfl_xor(acc[e], off);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Clock yardstick: each of 256 one-wave workgroups reads the shader-cycle
// counter and the constant-rate real-time counter, waits until the real-time
// counter has advanced by `ticks`, reads both again and writes the two
// differences (lane 0, ordinary vector stores).  Their ratio is the shader
// clock over the real-time counter's rate, at the moment the probe runs.
// A read of the real-time counter takes tens of shader cycles and the
// counter runs far slower than the shader clock, so the wait needs fewer
// than `ticks` reads; it stops after 64 * ticks + 65536 reads in any case.
constexpr int kClockProbeBlocks = 256;
__global__ __launch_bounds__(64) void clock_kernel(int64_t ticks, uint64_t* out) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r1 = r0;
  const uint64_t cap = 64 * (uint64_t)ticks + 65536;
  for (uint64_t i = 0; r1 - r0 < (uint64_t)ticks && i < cap; ++i)
    r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Matrix-core yardstick: every wave of 256 workgroups x 4 waves (one per
// SIMD) runs `iters` rounds of matrix-core products, 1024 cycles of them per
// round -- 64 v_mfma_f32_16x16x32 on 64 accumulators for 16-bit types, 32
// v_mfma_f32_16x16x4_f32 on 16 accumulators for binary32: the instructions
// the GEMM kernels issue -- on operand registers taken from caller data,
// nothing else in the loop; each thread then writes sums of its accumulators
// (so no product is dead).  Timing it gives the rate the matrix cores sustain
// on this part under the same data and power conditions as the GEMM.
constexpr int kMfmaProbeBlocks = 256;
template <int DT>
__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(const trt::u32x4* __restrict__ src,
                                                           int iters, trt::f32x16* sink) {
  const int t = threadIdx.x, lane = t & 63;
  trt::u32x4 a[4], b[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[i * 64 + lane];
    b[i] = src[256 + i * 64 + lane];
    a1[i] = src[512 + i * 64 + lane];
    b1[i] = src[768 + i * 64 + lane];
  }
  if constexpr (DT == trt::DT_F32) {
    // 16 accumulators of 4 lanes' worth; element e of sum g collects
    // accumulator 4g + e's register sums
    trt::f32x4 acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = trt::f32x4{};
    // the element goes through a scalar first: a bit cast applied to a
    // vector subscript directly reads element 0 whatever the index
    auto f = [](trt::u32x4 v, int e) {
      const uint32_t w = v[e];
      return __builtin_bit_cast(float, w);
    };
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(f(b[q % 4], q / 4), f(a[q / 4], q % 4), acc[q], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(f(b1[q % 4], q / 4), f(a1[q / 4], q % 4), acc[q], 0, 0, 0);
    }
    trt::f32x16 out{};
#pragma unroll
    for (int q = 0; q < 16; ++q)
      out[q] = acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3];
    sink[(int64_t)blockIdx.x * 256 + t] = out;
    return;
  }
  // 16-bit types: operand words A[i] = a[i], a1[i-4] and B[j] = b[j],
  // b1[j-4]; product q = 8i + j updates accumulator q; element e of the
  // sums collects the register sums of accumulators q with q % 16 == e
  const trt::u32x4 A[8] = {a[0], a[1], a[2], a[3], a1[0], a1[1], a1[2], a1[3]};
  const trt::u32x4 B[8] = {b[0], b[1], b[2], b[3], b1[0], b1[1], b1[2], b1[3]};
  trt::f32x4 acc[64];
#pragma unroll
  for (int q = 0; q < 64; ++q) acc[q] = trt::f32x4{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 64; ++q) acc[q] = trt::mfma16<DT>(B[q % 8], A[q / 8], acc[q]);
  }
  trt::f32x16 out{};
#pragma unroll
  for (int q = 0; q < 64; ++q) out[q % 16] += acc[q][0] + acc[q][1] + acc[q][2] + acc[q][3];
  sink[(int64_t)blockIdx.x * 256 + t] = out;
}

// ---- the layout algebra on caller arrays (host only) ------------------------

namespace {

// A caller's map: nin columns, each within nout bits.
trt_status read_lin(int32_t nin, int32_t nout, const uint32_t* cols, trt::gf2::Lin& l,
                    const char* what) {
  if (nin < 0 || nin > 32 || nout < 0 || nout > 32)
    return fail(TRT_ERR_ARG, std::string(what) + ": bit counts must be in [0, 32]");
  if (nin > 0 && !cols) return fail(TRT_ERR_NULL, std::string(what) + ": columns must be non-null");
  l = trt::gf2::zero(nin, nout);
  for (int i = 0; i < nin; ++i) {
    if (cols[i] & ~l.out_mask())
      return fail(TRT_ERR_ARG, std::string(what) + ": a column has bits beyond nout");
    l.col[i] = cols[i];
  }
  return TRT_OK;
}

void write_lin(const trt::gf2::Lin& l, uint32_t* out) {
  for (int i = 0; i < l.nin; ++i) out[i] = l.col[i];
}

}  // namespace

extern "C" {

int32_t trt_gf2_rank(int32_t nin, int32_t nout, const uint32_t* cols) {
  trt::gf2::Lin l{};
  if (read_lin(nin, nout, cols, l, "map") != TRT_OK) return -1;
  g_err.clear();
  return trt::gf2::rank(l);
}

trt_status trt_gf2_compose(int32_t outer_nin, int32_t outer_nout, const uint32_t* outer,
                           int32_t inner_nin, int32_t inner_nout, const uint32_t* inner,
                           uint32_t* out) {
  trt::gf2::Lin o{}, i{};
  if (const trt_status st = read_lin(outer_nin, outer_nout, outer, o, "outer"); st != TRT_OK) return st;
  if (const trt_status st = read_lin(inner_nin, inner_nout, inner, i, "inner"); st != TRT_OK) return st;
  if (outer_nin != inner_nout) return fail(TRT_ERR_ARG, "outer input bits must equal inner output bits");
  if (inner_nin > 0 && !out) return fail(TRT_ERR_NULL, "out must be non-null");
  write_lin(trt::gf2::compose(o, i), out);
  g_err.clear();
  return TRT_OK;
}

trt_status trt_gf2_product(int32_t a_nin, int32_t a_nout, const uint32_t* a, int32_t b_nin,
                           int32_t b_nout, const uint32_t* b, uint32_t* out) {
  trt::gf2::Lin la{}, lb{};
  if (const trt_status st = read_lin(a_nin, a_nout, a, la, "a"); st != TRT_OK) return st;
  if (const trt_status st = read_lin(b_nin, b_nout, b, lb, "b"); st != TRT_OK) return st;
  if (a_nin + b_nin > 32 || a_nout + b_nout > 32)
    return fail(TRT_ERR_SIZE, "the product has more than 32 input or output bits");
  if (a_nin + b_nin > 0 && !out) return fail(TRT_ERR_NULL, "out must be non-null");
  write_lin(trt::gf2::product(la, lb), out);
  g_err.clear();
  return TRT_OK;
}

trt_status trt_gf2_sublayout(int32_t nin, int32_t nout, const uint32_t* cols, uint32_t in_mask,
                             uint32_t out_mask, uint32_t* out, int32_t* out_nin,
                             int32_t* out_nout) {
  trt::gf2::Lin l{};
  if (const trt_status st = read_lin(nin, nout, cols, l, "map"); st != TRT_OK) return st;
  const trt::gf2::Lin r = trt::gf2::sublayout(l, in_mask, out_mask);
  if (r.nin > 0 && !out) return fail(TRT_ERR_NULL, "out must be non-null");
  write_lin(r, out);
  if (out_nin) *out_nin = r.nin;
  if (out_nout) *out_nout = r.nout;
  g_err.clear();
  return TRT_OK;
}

trt_status trt_gf2_invert_and_compose(int32_t r_nin, int32_t t_bits, const uint32_t* r,
                                      int32_t s_nin, const uint32_t* s, uint32_t* q) {
  trt::gf2::Lin lr{}, ls{}, lq{};
  if (const trt_status st = read_lin(r_nin, t_bits, r, lr, "R"); st != TRT_OK) return st;
  if (const trt_status st = read_lin(s_nin, t_bits, s, ls, "S"); st != TRT_OK) return st;
  if (r_nin > 0 && !q) return fail(TRT_ERR_NULL, "q must be non-null");
  if (!trt::gf2::invert_and_compose(lr, ls, lq))
    return fail(TRT_ERR_ARG, "a value of R is not a value of S");
  write_lin(lq, q);
  g_err.clear();
  return TRT_OK;
}

}  // extern "C"

extern "C" {

trt_status trt_validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int32_t opA,
                        const void* B, int64_t ldb, int32_t opB, const void* C, int64_t ldc,
                        int32_t in_dtype, int32_t out_dtype, const trt_epilogue* epi,
                        const trt_tile* tile) {
  std::string msg;
  const trt_status s = trt::validate_gemm(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                                          out_dtype, epi, msg);
  if (s != TRT_OK) return fail(s, msg);
  if (in_dtype == TRT_F32) {
    // binary32 operands run on one tile of their own
    if (tile && !(tile->bm == 128 && tile->bn == 128 && tile->bk == 32))
      return fail(TRT_ERR_UNSUPPORTED, "binary32 operands run on the 128x128x32 tile only");
  } else if (tile && !find_tile(tile)) {
    return fail(TRT_ERR_UNSUPPORTED, "no compiled kernel for the requested tile");
  }
  // one workgroup per output tile, counted in 32 bits by the launch
  const TileEntry* e = in_dtype == TRT_F32 ? nullptr : (tile ? find_tile(tile) : choose_tile(M, N));
  const int64_t bm = e ? e->bm : 128, bn = e ? e->bn : 128;
  if (((M + bm - 1) / bm) * ((N + bn - 1) / bn) > INT32_MAX)
    return fail(TRT_ERR_SIZE, "more than 2^31-1 output tiles in one launch");
  g_err.clear();
  return TRT_OK;
}

}  // extern "C"

namespace {

// Whether a call may split K over workgroups with a workspace, judged on
// sizes and storage alone: the streaming tile's kernel conditions without
// the pointers' alignment (checked at the call).
bool split_candidate(int64_t M, int64_t N, int64_t K, int32_t opA, int32_t opB,
                     int32_t in_dtype) {
  return M <= 16 && opA == TRT_OP_N && opB == TRT_OP_N && in_dtype != TRT_F32 && K % 8 == 0 &&
         N % 4 == 0;
}

// The workspace a call uses: the split plan's when it splits, else none.
int64_t workspace_need(int64_t M, int64_t N, int64_t K, int32_t opA, int32_t opB,
                       int32_t in_dtype) {
  if (!split_candidate(M, N, K, opA, opB, in_dtype)) return 0;
  return trt::skinny_split_plan(M, N, K).ws_bytes;
}

// The GEMM call behind trt_gemm, trt_gemm_tiled and trt_gemm_ws.  ws: the
// caller's workspace (use_ws), used to split K over workgroups for M <= 16
// when the streaming kernel applies; otherwise the same kernels as without.
trt_status gemm_call(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int32_t opA,
                     const void* B, int64_t ldb, int32_t opB, void* C, int64_t ldc,
                     int32_t in_dtype, int32_t out_dtype, const trt_epilogue* epi,
                     const trt_tile* tile, bool use_ws, void* ws, int64_t ws_bytes,
                     void* stream) {
  const trt_status s =
      trt_validate(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi, tile);
  if (s != TRT_OK) return s;
  const TileEntry* e = in_dtype == TRT_F32 ? nullptr : (tile ? find_tile(tile) : choose_tile(M, N));

  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.C = C;
  a.bias = epi ? epi->bias : nullptr;
  a.R = epi ? epi->residual : nullptr;
  a.scale = epi ? epi->row_scale : nullptr;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.ldr = (epi && epi->residual) ? epi->ldr : 0;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.relu = (epi && epi->relu) ? 1 : 0;
  a.out_dt = out_dtype;
  const int64_t isz = trt::elem_bytes(in_dtype);
  int64_t sa = 0, sb = 0;
  trt::span_bytes(opA ? K : M, opA ? M : K, lda, sa, isz);
  trt::span_bytes(opB ? N : K, opB ? K : N, ldb, sb, isz);
  a.a_bytes = sa;
  a.b_bytes = sb;
  // 16-byte operand vectors need 16-byte aligned bases and rows.
  const int64_t per16 = 16 / isz;
  const bool vec = aligned(A, 16) && aligned(B, 16) && lda % per16 == 0 && ldb % per16 == 0;
  // Epilogue vectors of 4 output elements (8 or 16 bytes) need aligned C,
  // bias and residual rows.
  const uintptr_t va = 4 * (uintptr_t)trt::elem_bytes(out_dtype);
  a.epi_vec = aligned(C, va) && ldc % 4 == 0 && (!a.bias || aligned(a.bias, va)) &&
              (!a.R || (aligned(a.R, va) && a.ldr % 4 == 0));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_ws && in_dtype != TRT_F32 && e->bm == 16 && skinny_ok(a, opA, opB)) {
    const trt::SplitPlan plan = trt::skinny_split_plan(M, N, K);
    if (plan.splits >= 2) {
      std::string msg;
      const trt_status w = trt::validate_workspace(M, N, K, A, lda, opA, B, ldb, opB, C, ldc,
                                                   in_dtype, out_dtype, epi, ws, ws_bytes,
                                                   plan.ws_bytes, msg);
      if (w != TRT_OK) return fail(w, msg);
      return launched(trt::launch_skinny_split(a, in_dtype, static_cast<float*>(ws), plan.splits,
                                               plan.per_split, st),
                      "gemm launch");
    }
  }
  return launched(in_dtype == TRT_F32 ? trt::launch_f32(a, opA, opB, vec, st)
                                      : e->launch(a, in_dtype, opA, opB, vec, st),
                  "gemm launch");
}

}  // namespace

extern "C" {

trt_status trt_gemm_tiled(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                          int32_t opA, const void* B, int64_t ldb, int32_t opB, void* C,
                          int64_t ldc, int32_t in_dtype, int32_t out_dtype,
                          const trt_epilogue* epi, const trt_tile* tile, void* stream) {
  return gemm_call(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi, tile,
                   false, nullptr, 0, stream);
}

int64_t trt_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t opA, int32_t opB,
                                int32_t in_dtype) {
  if (M < 1 || N < 1 || K < 1 || M > trt::kMaxDim || N > trt::kMaxDim || K > trt::kMaxDim) {
    fail(TRT_ERR_SIZE, "M, N and K must be in [1, 2^30]");
    return -1;
  }
  if ((opA != TRT_OP_N && opA != TRT_OP_T) || (opB != TRT_OP_N && opB != TRT_OP_T)) {
    fail(TRT_ERR_ARG, "opA and opB must be TRT_OP_N or TRT_OP_T");
    return -1;
  }
  if (in_dtype != TRT_F16 && in_dtype != TRT_BF16 && in_dtype != TRT_F32) {
    fail(TRT_ERR_DTYPE, "in_dtype must be TRT_F16, TRT_BF16 or TRT_F32");
    return -1;
  }
  g_err.clear();
  return workspace_need(M, N, K, opA, opB, in_dtype);
}

trt_status trt_gemm_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int32_t opA,
                       const void* B, int64_t ldb, int32_t opB, void* C, int64_t ldc,
                       int32_t in_dtype, int32_t out_dtype, const trt_epilogue* epi,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_call(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi, nullptr,
                   true, workspace, workspace_bytes, stream);
}

trt_status trt_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int32_t opA,
                    const void* B, int64_t ldb, int32_t opB, void* C, int64_t ldc,
                    int32_t in_dtype, int32_t out_dtype, const trt_epilogue* epi, void* stream) {
  return trt_gemm_tiled(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi,
                        nullptr, stream);
}

trt_status trt_choose_tile(int64_t M, int64_t N, int32_t in_dtype, trt_tile* tile) {
  if (!tile) return fail(TRT_ERR_NULL, "tile must be non-null");
  if (M < 1 || N < 1 || M > trt::kMaxDim || N > trt::kMaxDim)
    return fail(TRT_ERR_SIZE, "M and N must be in [1, 2^30]");
  if (in_dtype != TRT_F16 && in_dtype != TRT_BF16 && in_dtype != TRT_F32)
    return fail(TRT_ERR_DTYPE, "in_dtype must be TRT_F16, TRT_BF16 or TRT_F32");
  if (in_dtype == TRT_F32) {
    *tile = trt_tile{128, 128, 32};
  } else {
    const TileEntry* e = choose_tile(M, N);
    *tile = trt_tile{e->bm, e->bn, e->bk};
  }
  g_err.clear();
  return TRT_OK;
}

int32_t trt_tile_count(void) { return kNumTiles; }

trt_status trt_tile_at(int32_t i, trt_tile* tile, int32_t* waves_m, int32_t* waves_n,
                       int32_t* regs_per_lane, int32_t* frag) {
  if (i < 0 || i >= kNumTiles) return fail(TRT_ERR_ARG, "tile index out of range");
  const TileEntry& e = kTiles[i];
  if (tile) *tile = trt_tile{e.bm, e.bn, e.bk};
  if (waves_m) *waves_m = e.wm;
  if (waves_n) *waves_n = e.wn;
  if (regs_per_lane) *regs_per_lane = e.regs;
  if (frag) *frag = e.frag;
  g_err.clear();
  return TRT_OK;
}

int64_t trt_layout_size(int32_t map_id, const trt_tile* tile) {
  if (!tile) return -1;
  const TileEntry* e = find_tile(tile);
  return e ? e->size(map_id) : -1;
}

trt_status trt_layout_dump_host(int32_t map_id, const trt_tile* tile, int32_t* rows,
                                int32_t* cols, int64_t n) {
  if (!tile) return fail(TRT_ERR_NULL, "tile must be non-null");
  const TileEntry* e = find_tile(tile);
  if (!e) return fail(TRT_ERR_UNSUPPORTED, "no compiled kernel for the requested tile");
  const int64_t size = e->size(map_id);
  if (size < 0) return fail(TRT_ERR_ARG, "unknown map id");
  if (n != size) return fail(TRT_ERR_SIZE, "n must equal trt_layout_size(map_id, tile)");
  if (!rows || !cols) return fail(TRT_ERR_NULL, "rows and cols must be non-null");
  for (int64_t x = 0; x < n; ++x) {
    int r, c;
    e->eval(map_id, x, r, c);
    rows[x] = r;
    cols[x] = c;
  }
  g_err.clear();
  return TRT_OK;
}

trt_status trt_layout_dump(int32_t map_id, const trt_tile* tile, int32_t* rows, int32_t* cols,
                           int64_t n, void* stream) {
  if (!tile) return fail(TRT_ERR_NULL, "tile must be non-null");
  const TileEntry* e = find_tile(tile);
  if (!e) return fail(TRT_ERR_UNSUPPORTED, "no compiled kernel for the requested tile");
  const int64_t size = e->size(map_id);
  if (size < 0) return fail(TRT_ERR_ARG, "unknown map id");
  if (n != size) return fail(TRT_ERR_SIZE, "n must equal trt_layout_size(map_id, tile)");
  if (!rows || !cols) return fail(TRT_ERR_NULL, "rows and cols must be non-null");
  return launched(e->dump(map_id, rows, cols, n, static_cast<hipStream_t>(stream)),
                  "layout dump launch");
}

trt_status trt_layout_rank(const trt_tile* tile, int32_t* rank, int32_t* in_bits,
                           int32_t* out_bits) {
  if (!tile) return fail(TRT_ERR_NULL, "tile must be non-null");
  const TileEntry* e = find_tile(tile);
  if (!e) return fail(TRT_ERR_UNSUPPORTED, "no compiled kernel for the requested tile");
  if (e->rank < 0)
    return fail(TRT_ERR_UNSUPPORTED,
                "this tile's ownership is integer-affine, not GF(2)-linear; it has no rank");
  if (rank) *rank = e->rank;
  if (in_bits) *in_bits = e->in_bits;
  if (out_bits) *out_bits = e->out_bits;
  g_err.clear();
  return TRT_OK;
}

trt_status trt_mfma_probe(int32_t dtype, int32_t shape, const void* a, const void* b, float* c,
                          void* stream) {
  if (!a || !b || !c) return fail(TRT_ERR_NULL, "a, b and c must be non-null");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16))
    return fail(TRT_ERR_ALIGN, "a, b and c must be 16-byte aligned");
  if (dtype != TRT_F16 && dtype != TRT_BF16)
    return fail(TRT_ERR_DTYPE, "dtype must be TRT_F16 or TRT_BF16");
  if (shape != 16 && shape != 32) return fail(TRT_ERR_ARG, "shape must be 16 or 32");
  const auto* av = static_cast<const trt::u32x4*>(a);
  const auto* bv = static_cast<const trt::u32x4*>(b);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (shape == 16) {
    auto* cv = reinterpret_cast<trt::f32x4*>(c);
    e = dtype == TRT_F16 ? trt::launch(probe_kernel<trt::DT_F16>, dim3(1), dim3(64), 0, s, av, bv, cv)
                         : trt::launch(probe_kernel<trt::DT_BF16>, dim3(1), dim3(64), 0, s, av, bv, cv);
  } else {
    auto* cv = reinterpret_cast<trt::f32x16*>(c);
    e = dtype == TRT_F16
            ? trt::launch(probe32_kernel<trt::DT_F16>, dim3(1), dim3(64), 0, s, av, bv, cv)
            : trt::launch(probe32_kernel<trt::DT_BF16>, dim3(1), dim3(64), 0, s, av, bv, cv);
  }
  return launched(e, "probe launch");
}

trt_status trt_hbm_read_probe(const void* x, int64_t bytes, void* sink, int64_t sink_bytes,
                              void* stream) {
  if (!x || !sink) return fail(TRT_ERR_NULL, "x and sink must be non-null");
  if (bytes < 16 || bytes % 16 != 0)
    return fail(TRT_ERR_SIZE, "bytes must be a positive multiple of 16");
  if (sink_bytes < TRT_READ_PROBE_SINK_BYTES)
    return fail(TRT_ERR_SIZE, "sink must hold TRT_READ_PROBE_SINK_BYTES bytes");
  if (!aligned(x, 16) || !aligned(sink, 16))
    return fail(TRT_ERR_ALIGN, "x and sink must be 16-byte aligned");
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), s0 = reinterpret_cast<uintptr_t>(sink);
  if (x0 < s0 + (uintptr_t)TRT_READ_PROBE_SINK_BYTES && s0 < x0 + (uintptr_t)bytes)
    return fail(TRT_ERR_OVERLAP, "sink must not overlap x");
  static_assert(kReadProbeBlocks * 16 == TRT_READ_PROBE_SINK_BYTES, "one digest per workgroup");
  return launched(trt::launch(hbm_read_kernel, dim3(kReadProbeBlocks), dim3(256), 0,
                              static_cast<hipStream_t>(stream),
                              static_cast<const trt::u32x4*>(x), bytes / 16,
                              static_cast<trt::u32x4*>(sink)),
                  "read probe launch");
}

trt_status trt_mfma_loop_probe(int32_t dtype, const void* operands, int32_t iters, float* sink,
                               int64_t sink_bytes, void* stream) {
  if (!operands || !sink) return fail(TRT_ERR_NULL, "operands and sink must be non-null");
  if (dtype != TRT_F16 && dtype != TRT_BF16 && dtype != TRT_F32)
    return fail(TRT_ERR_DTYPE, "dtype must be TRT_F16, TRT_BF16 or TRT_F32");
  if (iters < 1) return fail(TRT_ERR_ARG, "iters must be positive");
  if (sink_bytes < TRT_MFMA_PROBE_SINK_BYTES)
    return fail(TRT_ERR_SIZE, "sink must hold TRT_MFMA_PROBE_SINK_BYTES bytes");
  if (!aligned(operands, 16) || !aligned(sink, 64))
    return fail(TRT_ERR_ALIGN, "operands must be 16-byte and sink 64-byte aligned");
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(operands), s0 = reinterpret_cast<uintptr_t>(sink);
  if (o0 < s0 + (uintptr_t)TRT_MFMA_PROBE_SINK_BYTES && s0 < o0 + (uintptr_t)TRT_MFMA_PROBE_OPERAND_BYTES)
    return fail(TRT_ERR_OVERLAP, "sink must not overlap the operands");
  static_assert(kMfmaProbeBlocks * 256 * 64 == TRT_MFMA_PROBE_SINK_BYTES, "one sum per thread");
  const auto* src = static_cast<const trt::u32x4*>(operands);
  auto* dst = reinterpret_cast<trt::f32x16*>(sink);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(kMfmaProbeBlocks), block(256);
  const hipError_t e =
      dtype == TRT_F16   ? trt::launch(mfma_loop_kernel<trt::DT_F16>, grid, block, 0, s, src, iters, dst)
      : dtype == TRT_F32 ? trt::launch(mfma_loop_kernel<trt::DT_F32>, grid, block, 0, s, src, iters, dst)
                         : trt::launch(mfma_loop_kernel<trt::DT_BF16>, grid, block, 0, s, src, iters, dst);
  return launched(e, "matrix-core probe launch");
}

trt_status trt_clock_probe(int64_t ticks, void* sink, int64_t sink_bytes, void* stream) {
  if (!sink) return fail(TRT_ERR_NULL, "sink must be non-null");
  if (ticks < 1 || ticks > (int64_t(1) << 27)) return fail(TRT_ERR_ARG, "ticks must be in [1, 2^27]");
  if (sink_bytes < TRT_CLOCK_PROBE_SINK_BYTES)
    return fail(TRT_ERR_SIZE, "sink must hold TRT_CLOCK_PROBE_SINK_BYTES bytes");
  if (!aligned(sink, 8)) return fail(TRT_ERR_ALIGN, "sink must be 8-byte aligned");
  static_assert(kClockProbeBlocks * 16 == TRT_CLOCK_PROBE_SINK_BYTES, "two counters per workgroup");
  return launched(trt::launch(clock_kernel, dim3(kClockProbeBlocks), dim3(64), 0,
                              static_cast<hipStream_t>(stream), ticks,
                              static_cast<uint64_t*>(sink)),
                  "clock probe launch");
}

trt_status trt_block_reduce(const void* x, int64_t n, int64_t block, int32_t dtype, int32_t op,
                            float* out, void* stream) {
  if (n < 1 || block < 1) return fail(TRT_ERR_SIZE, "n and block must be >= 1");
  if (n > (int64_t(1) << 40)) return fail(TRT_ERR_SIZE, "n must be <= 2^40");
  if (dtype != TRT_F16 && dtype != TRT_BF16 && dtype != TRT_F32)
    return fail(TRT_ERR_DTYPE, "dtype must be TRT_F16, TRT_BF16 or TRT_F32");
  if (op != TRT_REDUCE_SUM && op != TRT_REDUCE_MAX && op != TRT_REDUCE_MIN)
    return fail(TRT_ERR_ARG, "op must be TRT_REDUCE_SUM, TRT_REDUCE_MAX or TRT_REDUCE_MIN");
  if (!x || !out) return fail(TRT_ERR_NULL, "x and out must be non-null");
  const int64_t esz = trt::elem_bytes(dtype);
  if (!aligned(x, (uintptr_t)esz) || !aligned(out, 4))
    return fail(TRT_ERR_ALIGN, "x must be aligned to its element and out to 4 bytes");
  const int64_t nblocks = (n + block - 1) / block;
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), o0 = reinterpret_cast<uintptr_t>(out);
  if (x0 < o0 + (uintptr_t)(4 * nblocks) && o0 < x0 + (uintptr_t)(esz * n))
    return fail(TRT_ERR_OVERLAP, "out must not overlap x");
  trt::ReduceArgs a{};
  a.x = x;
  a.out = out;
  a.n = n;
  a.block = block;
  a.nblocks = nblocks;
  a.vec = aligned(x, 16) && (block * esz) % 16 == 0;
  return launched(trt::launch_reduce(a, dtype, op, static_cast<hipStream_t>(stream)),
                  "block reduction launch");
}

trt_status trt_regtile_thread_shape(int32_t lm, int32_t ln, int32_t max_threads, int32_t* tm,
                                    int32_t* tn) {
  if (!tm || !tn) return fail(TRT_ERR_NULL, "tm and tn must be non-null");
  if (lm < 1 || ln < 1) return fail(TRT_ERR_SIZE, "lm and ln must be >= 1");
  if (max_threads < 1) return fail(TRT_ERR_ARG, "max_threads must be >= 1");
  int a = 1, b = 1;
  trt::regtile_thread_shape(lm, ln, max_threads, a, b);
  *tm = a;
  *tn = b;
  g_err.clear();
  return TRT_OK;
}

trt_status trt_regtile_owner(int32_t lm, int32_t ln, int32_t tm, int32_t tn, int32_t* rows,
                             int32_t* cols, int64_t n) {
  if (lm < 1 || ln < 1 || tm < 1 || tn < 1)
    return fail(TRT_ERR_SIZE, "tile and thread shapes must be positive");
  if (lm % tm || ln % tn) return fail(TRT_ERR_ARG, "the thread shape must divide the tile");
  if ((int64_t)lm * ln > (int64_t(1) << 24)) return fail(TRT_ERR_SIZE, "lm * ln must be <= 2^24");
  if (n != (int64_t)lm * ln) return fail(TRT_ERR_SIZE, "n must equal lm * ln");
  if (!rows || !cols) return fail(TRT_ERR_NULL, "rows and cols must be non-null");
  const int regs = (lm / tm) * (ln / tn), rn = ln / tn;
  std::vector<uint8_t> seen((size_t)n, 0);
  for (int t = 0; t < tm * tn; ++t)
    for (int r = 0; r < regs; ++r) {
      int row, col;
      trt::regtile_coord(t, r, tm, tn, rn, row, col);
      const int64_t x = (int64_t)t * regs + r;
      rows[x] = row;
      cols[x] = col;
      if (row < 0 || row >= lm || col < 0 || col >= ln || seen[(size_t)row * ln + col]++)
        return fail(TRT_ERR_ARG, "ownership is not exactly once");
    }
  g_err.clear();
  return TRT_OK;
}

trt_status trt_gemm_regtile(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            int32_t opA, const void* B, int64_t ldb, int32_t opB, void* C,
                            int64_t ldc, int32_t in_dtype, int32_t out_dtype,
                            const trt_epilogue* epi, int32_t lm, int32_t ln,
                            int32_t max_threads, void* stream) {
  std::string msg;
  const trt_status s = trt::validate_gemm(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype,
                                          out_dtype, epi, msg);
  if (s != TRT_OK) return fail(s, msg);
  if (lm < 1 || ln < 1) return fail(TRT_ERR_SIZE, "lm and ln must be >= 1");
  if (max_threads < 1 || max_threads > trt::kRegtileThreads)
    return fail(TRT_ERR_ARG, "max_threads must be in [1, 64]");
  int tm = 1, tn = 1;
  trt::regtile_thread_shape(lm, ln, max_threads, tm, tn);
  if (lm / tm > trt::kRegtileMaxRegs || ln / tn > trt::kRegtileMaxRegs)
    return fail(TRT_ERR_UNSUPPORTED, "more than 8 registers per axis for this tile");
  if (((M + lm - 1) / lm) * ((N + ln - 1) / ln) > INT32_MAX)
    return fail(TRT_ERR_SIZE, "more than 2^31-1 output tiles in one launch");
  trt::RegtileArgs a{};
  a.g.A = static_cast<const uint16_t*>(A);
  a.g.B = static_cast<const uint16_t*>(B);
  a.g.C = C;
  a.g.bias = epi ? epi->bias : nullptr;
  a.g.R = epi ? epi->residual : nullptr;
  a.g.scale = epi ? epi->row_scale : nullptr;
  a.g.lda = lda;
  a.g.ldb = ldb;
  a.g.ldc = ldc;
  a.g.ldr = (epi && epi->residual) ? epi->ldr : 0;
  a.g.M = (int32_t)M;
  a.g.N = (int32_t)N;
  a.g.K = (int32_t)K;
  a.g.relu = (epi && epi->relu) ? 1 : 0;
  a.g.out_dt = out_dtype;
  a.lm = lm;
  a.ln = ln;
  a.tm = tm;
  a.tn = tn;
  a.rm = lm / tm;
  a.rn = ln / tn;
  a.opA = opA;
  a.opB = opB;
  const int64_t isz = trt::elem_bytes(in_dtype);
  int64_t sa = 0, sb = 0;
  trt::span_bytes(opA ? K : M, opA ? M : K, lda, sa, isz);
  trt::span_bytes(opB ? N : K, opB ? K : N, ldb, sb, isz);
  a.g.a_bytes = sa;
  a.g.b_bytes = sb;
  return launched(trt::launch_regtile(a, in_dtype, static_cast<hipStream_t>(stream)),
                  "register-tile gemm launch");
}

}  // extern "C"

// ---- the allocation-free variant of trt_gemm_ws --------------------------------
//
// Its workspace is this array, one per device, in the library's code object
// (no allocation by anyone).  Host code never passes the array's name to a
// kernel: that is a host-side stand-in, not a device address.  The device
// address is looked up once per device, with that device current, and
// passed to the kernels like a caller's workspace.
static __device__ __align__(256) char scratch[TRT_NOALLOC_SCRATCH_BYTES];

namespace {

// Every split plan fits the array: M <= 16 rows, and for p column panels a
// plan takes at most ceil(512 / p) slices (fewer when K is short), so its
// workspace is at most 16 * 4 * 256 p * ceil(512 / p) bytes over all p.
constexpr bool scratch_fits_every_plan() {
  for (int64_t p = 1; p <= 4096; ++p)
    if (trt::skinny_split_plan(16, 256 * p, int64_t(1) << 30).ws_bytes > TRT_NOALLOC_SCRATCH_BYTES)
      return false;
  return true;
}
static_assert(scratch_fits_every_plan(), "the scratch array holds every split plan's workspace");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of device dev's scratch array, looked up on first use
// with dev current (the caller's current device is restored).
trt_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(TRT_ERR_ARG, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !ptr)
      return fail(TRT_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return TRT_OK;
}

}  // namespace

extern "C" {

trt_status trt_gemm_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            int32_t opA, const void* B, int64_t ldb, int32_t opB, void* C,
                            int64_t ldc, int32_t in_dtype, int32_t out_dtype,
                            const trt_epilogue* epi, void* stream) {
  const trt_status s =
      trt_validate(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi, nullptr);
  if (s != TRT_OK) return s;
  const int64_t need = workspace_need(M, N, K, opA, opB, in_dtype);
  if (need > TRT_NOALLOC_SCRATCH_BYTES)
    return fail(TRT_ERR_SIZE, "this call needs " + std::to_string(need) +
                                  " bytes of workspace, more than the " +
                                  std::to_string((int64_t)TRT_NOALLOC_SCRATCH_BYTES) +
                                  " of the allocation-free variant; use trt_gemm_ws");
  void* ws = nullptr;
  if (need > 0) {
    // the device the stream runs on
    int dev = -1;
    const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return fail(TRT_ERR_HIP, std::string("stream device: ") + hipGetErrorString(e));
    const trt_status a = scratch_address(dev, &ws);
    if (a != TRT_OK) return a;
  }
  return gemm_call(M, N, K, A, lda, opA, B, ldb, opB, C, ldc, in_dtype, out_dtype, epi, nullptr,
                   true, ws, need > 0 ? TRT_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int32_t trt_abi_version(void) { return TRT_ABI_VERSION; }

const char* trt_last_error(void) { return g_err.c_str(); }

}  // extern "C"
