// gemm_f32_dma.hpp -- the binary32 GEMM with direct-to-LDS copies, for gfx950.
//
// Same tile, fragments, products and epilogue as gemm_f32_kernel (128x128
// tile with a K step of 32, 2x2 waves of 64x64, v_mfma_f32_16x16x4_f32 with
// lane group g taking k = 8g + kk at product step kk), so the two kernels
// compute bit-identical results.  The operand tiles travel differently:
// every 16-byte chunk goes from global memory straight into LDS
// (buffer_load ... lds, as in the 16-bit pipelined kernel): no staging
// registers, no register transposes, no LDS store instructions.  Two LDS
// stages of 32 KiB; the copies of step kt+1 are issued during step kt and
// awaited at its end, so two workgroups share a compute unit.
//
// LDS layouts, one 16 KiB region per operand and stage:
//   k-contiguous storage (A row-major, B^T): [128 rows][32 k], chunk kc (k
//     4kc..4kc+3) of row r at chunk position kc ^ f32_swz(r), read as two
//     16-byte loads per fragment row (the binary32 kernel's layout);
//   rows-contiguous storage (B row-major, A^T): [32 k][128 rows], the
//     natural layout of the global rows, with 16-float blocks of row k
//     XOR-ed by 16 * ((k >> 3) & 3).  A lane of group g reads its four k
//     = 8g + 4h + e (e = 0..3) of column c as four 4-byte loads 512 bytes
//     apart; the 64 lanes of one load touch row k = 8g + 4h + e at float
//     (c ^ 16g), i.e. 64 distinct banks.
// Lane t of wave instruction i fills chunk slot s = 256 i + t of a region
// and fetches the chunk that slot holds; both slot maps are bijections,
// checked at compile time.
//
// Bounds: a buffer descriptor per operand and K step whose record count is
// what is left of the operand; a chunk past it reads zero.  The caller
// guarantees that no chunk straddles the end: K % 4 == 0 for k-contiguous
// operands, rows % 4 == 0 for rows-contiguous ones.  Rows beyond M or N only
// feed accumulators the epilogue never stores; on a partial last K step the
// k-contiguous chunks at k >= K are forced out of range, and rows-contiguous
// rows k >= K lie past the operand's end.
#pragma once

#include "gemm_dma.hpp"
#include "gemm_f32.hpp"

namespace trt {

struct F32DmaLayout {
  static constexpr int R = 128;             // rows (m or n) per tile
  static constexpr int CHUNKS = R * 32 / 4; // 16-byte chunks per region
  static constexpr int NCH = CHUNKS / 256;  // copies per thread per stage
  static constexpr int BYTES = R * 32 * 4;  // one region

  // k-contiguous: slot s -> (row, chunk of k)
  static constexpr int kc_row(int s) { return s / 8; }
  static constexpr int kc_chunk(int s) { return (s % 8) ^ (((s / 8) ^ (s / 8 >> 3)) & 7); }
  // rows-contiguous: slot s -> (k, chunk of 4 rows)
  static constexpr int mn_k(int s) { return s / 32; }
  static constexpr int mn_chunk(int s) { return (s % 32) ^ (4 * ((s / 32 >> 3) & 3)); }

  // Every (row, chunk) of a region filled by exactly one slot.
  static constexpr bool bijective(bool kc) {
    bool seen[CHUNKS] = {};
    for (int s = 0; s < CHUNKS; ++s) {
      const int cell = kc ? kc_row(s) * 8 + kc_chunk(s) : mn_k(s) * 32 + mn_chunk(s);
      if (cell < 0 || cell >= CHUNKS || seen[cell]) return false;
      seen[cell] = true;
    }
    return true;
  }
};
static_assert(F32DmaLayout::NCH * 256 == F32DmaLayout::CHUNKS, "whole copy rounds");
static_assert(F32DmaLayout::bijective(true) && F32DmaLayout::bijective(false),
              "copy slot maps cover each region exactly once");

// One operand's copies.  X row-major with leading dimension ld (elements):
// KC: element (r, k) at X[r*ld + k]; else at X[k*ld + r].
template <bool KC>
struct F32DmaOperand {
  using L = F32DmaLayout;
  const char* base;
  int64_t extent;       // bytes
  int64_t step_bytes;   // bytes per K step of 32
  uint32_t voff[L::NCH];
  int kfirst[L::NCH];   // KC: first k (within a step) of each chunk

  __device__ __forceinline__ void init(const float* X, int64_t ld, int64_t ext, int row0, int t) {
    base = reinterpret_cast<const char*>(X);
    extent = ext;
#pragma unroll
    for (int i = 0; i < L::NCH; ++i) {
      const int s = 256 * i + t;
      if (KC) {
        voff[i] = (uint32_t)(((int64_t)(row0 + L::kc_row(s)) * ld + 4 * L::kc_chunk(s)) * 4);
        kfirst[i] = 4 * L::kc_chunk(s);
      } else {
        voff[i] = (uint32_t)(((int64_t)L::mn_k(s) * ld + row0 + 4 * L::mn_chunk(s)) * 4);
        kfirst[i] = 0;
      }
    }
    step_bytes = KC ? 32 * 4 : 32 * 4 * ld;
  }

  // Descriptor of K step `step` of nk: zero records (nothing fetched) past
  // the operand's end and for the step after the last, whose copies the
  // last iteration issues.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int step, int nk) const {
    const int64_t adv = (int64_t)step * step_bytes;
    const bool live = step < nk && adv < extent;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (live ? adv : 0)), (short)0,
                                             live ? (int)(extent - adv) : 0, kBufferFormat);
  }

  // Copy i of K step `step` into the region at LDS byte address dst.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int step, uint32_t dst,
                                        int wave, int K, bool last_partial, int i) const {
    const bool drop = KC && last_partial && (step * 32 + kfirst[i] >= K);
    dma16(rs, __builtin_amdgcn_readfirstlane(dst + (256 * i + 64 * wave) * 16),
          drop ? 0x80000000u : voff[i]);
  }
};

// Four floats of a fragment: k = 8g + 4h + e (e = 0..3) of fragment row
// `row`, for lane group g, from one operand region.
template <bool KC>
__device__ __forceinline__ f32x4 f32_frag(const TRT_LDS float* region, int row, int g, int h) {
  if constexpr (KC) {
    return *(const TRT_LDS f32x4*)(region + f32_slot(row, 2 * g + h));
  } else {
    const TRT_LDS float* p = region + (8 * g + 4 * h) * 128 + (row ^ (16 * g));
    return f32x4{p[0], p[128], p[256], p[384]};
  }
}

template <bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void gemm_f32_dma_kernel(GemmArgs p) {
  using TL = TileF32;
  using L = F32DmaLayout;
  constexpr int FM = TL::FM, FN = TL::FN;
  static_assert(TL::BM == L::R && TL::BN == L::R && TL::THREADS == 256 && FM == 4 && FN == 4,
                "128x128 tile, 4 waves of 4x4 fragments");
  constexpr int STAGE = 2 * L::BYTES;
  constexpr int LOADS = 2 * L::NCH;
  static_assert(LOADS == 8, "one copy every four of the first 32 products");
  __shared__ __attribute__((aligned(1024))) float lds_raw[2 * STAGE / 4];
  TRT_LDS float* lds = (TRT_LDS float*)lds_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int tm, tn;
  tile_of<8>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * TL::BM, n0 = tn * TL::BN;

  F32DmaOperand<A_KC> a;
  F32DmaOperand<B_KC> b;
  a.init(reinterpret_cast<const float*>(p.A), p.lda, p.a_bytes, m0, t);
  b.init(reinterpret_cast<const float*>(p.B), p.ldb, p.b_bytes, n0, t);
  const int nk = (p.K + 31) / 32;
  const bool partial = (p.K & 31) != 0;

  const int wrow = (wave / TL::WN) * TL::WTM, wcol = (wave % TL::WN) * TL::WTN;
  const int fr = lane & 15, g = lane >> 4;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto copy = [&](__amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb, int step, int c) {
    const uint32_t st = lds_base + (step & 1) * STAGE;
    const bool lp = partial && step == nk - 1;
    if (c < L::NCH) a.issue(rsa, step, st, wave, p.K, lp, c);
    else b.issue(rsb, step, st + L::BYTES, wave, p.K, lp, c - L::NCH);
  };
  {
    const auto rsa = a.rsrc(0, nk), rsb = b.rsrc(0, nk);
#pragma unroll
    for (int c = 0; c < LOADS; ++c) copy(rsa, rsb, 0, c);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Per K step: the first half's fragments are read; the first half's 64
  // products run with the second half's fragment reads (in its first eight
  // products) and this thread's copies of step kt+1 (one every four
  // products among the first 32 -- early, so that they have most of the
  // step to land; 1.3 % faster than one every eight over all 64 -- into the
  // other stage, last read before the previous barrier) in a fixed order; then the second half's 64 products; then the wait for
  // the copies and the barrier.  The last step's copies (of step nk) read
  // zeros into the stage that no later step reads.
  for (int kt = 0; kt < nk; ++kt) {
    const TRT_LDS float* la = lds + (kt & 1) * (STAGE / 4);
    const TRT_LDS float* lb = la + L::BYTES / 4;
    const auto rsa = a.rsrc(kt + 1, nk), rsb = b.rsrc(kt + 1, nk);
    f32x4 af[FM][2], bf[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i][0] = f32_frag<A_KC>(la, wrow + 16 * i + fr, g, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j][0] = f32_frag<B_KC>(lb, wcol + 16 * j + fr, g, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 64; ++q) {
      const int kk = q / 16, i = (q / 4) % 4, j = q % 4;
      acc[i][j] = mfma16_f32(bf[j][0][kk], af[i][0][kk], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (q < FM) af[q][1] = f32_frag<A_KC>(la, wrow + 16 * q + fr, g, 1);
      else if (q < FM + FN) bf[q - FM][1] = f32_frag<B_KC>(lb, wcol + 16 * (q - FM) + fr, g, 1);
      if (q % 4 == 1 && q < 32) copy(rsa, rsb, kt + 1, q / 4);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16_f32(bf[j][1][kk], af[i][1][kk], acc[i][j]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  epilogue_store<TL>(p, acc, m0, n0, lane, wave);
}

}  // namespace trt
