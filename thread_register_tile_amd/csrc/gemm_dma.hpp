// gemm_dma.hpp -- the pipelined main-path GEMM kernel for gfx950.
//
// Same contract as the generic kernel in gemm_kernel.hpp, with 16x16x32
// matrix-core fragments (the tile's ownership map is stated in layout.hpp).
// It differs in how operand tiles reach the matrix cores:
//
//   * Direct-to-LDS copies.  Each 16-byte chunk goes from global memory
//     straight into LDS (buffer_load ... lds): no staging registers, no LDS
//     store instructions.  A wave instruction fills 64 consecutive LDS slots,
//     so each lane fetches the chunk its slot holds under the XOR swizzle.
//   * Hardware bounds.  Each operand is read through a buffer descriptor whose
//     record count is the operand's byte extent, rebased every K step: a copy
//     reaching past the extent returns zero and never faults.  The check
//     covers a 16-byte copy as a whole, so the caller guarantees that no copy
//     straddles the extent's end (K % 8 == 0 for k-contiguous operands, rows
//     % 8 == 0 for rows-contiguous ones).  Rows beyond M or N are read (or
//     zero) but only feed accumulators the epilogue never stores; k beyond K
//     reads zero for rows-contiguous operands and is forced out of range for
//     k-contiguous chunks on the last, partial K step.
//   * Transposing fragment reads.  A rows-contiguous operand (row-major B, or
//     A^T) keeps its natural [k][rows] layout in LDS and reaches the matrix
//     core through ds_read_b64_tr_b16: within each 16 lanes, output lane i,
//     element v is input lane 4v + i/4, element i%4.  Lanes 4v..4v+3 read k row
//     k0+v at columns c0, c0+4, c0+8, c0+12, so output lane i holds k0..k0+3
//     of column c0+i -- the matrix-core operand layout, two reads per 8 k.
//   * Four LDS stages of one 32-wide K step each (4 x 32 KiB), copies issued
//     three steps ahead, one barrier per step.
//   * 16x16x32 products: one product consumes the whole 32-wide K step, and
//     moves half the accumulator bytes per FLOP of the 32x32x16 shape (4
//     result registers per 16 cycles instead of 16 per 32); under the power
//     limit the matrix cores sustain a higher rate with it (measured 1950 vs
//     1700 TFLOP/s in a products-only loop on the same data), and the GEMM
//     gains 3-8 % across storage orders.
//
// Per K step kt, per wave, one block of FM x FN products on one set of
// operand registers:
//   the first half (fragment rows 0..FM/2-1 against every column, column by
//   column), with this thread's copies of step kt+3 into stage (kt+3)%4
//   and the reads of step kt's fragment rows FM/2..FM-1 spread through it;
//   wait for this wave's LDS reads and for its copies of step kt+1;
//   workgroup barrier;
//   the second half (rows FM/2..FM-1, column by column), refilling the
//   operand registers with step kt+1's fragments as they die: rows
//   0..FM/2-1 first, each column after its last product.
// Stage (kt+3)%4 was last read by reads issued in step kt-2 and in the first
// half of step kt-1, completed before the barrier of step kt-1, which
// precedes the copies of step kt; the copies of step kt+1 are complete and
// visible once every wave has waited for its own and passed the barrier of
// step kt.
#pragma once

#include "gemm_kernel.hpp"

namespace trt {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define TRT_LDS __attribute__((address_space(3)))

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector memory
// operations (or n LDS operations) of this wave are outstanding.
constexpr int waitcnt_vm(int n) { return ((n >> 4) & 3) << 14 | 0x0F70 | (n & 15); }
constexpr int waitcnt_lgkm(int n) { return 0xC07F | ((n & 15) << 8); }

// One 16-byte direct-to-LDS copy per lane: global (buffer) byte offset voff
// -> LDS byte address lds_addr + 16 * lane.  lds_addr is wave-uniform (it
// travels in M0).  Written as inline assembly so that the compiler does not
// treat the copy as a pending LDS store that every later LDS read must wait
// for: the kernel orders copies and reads itself with s_waitcnt vmcnt and
// barriers.  M0 is saved and restored around the copy.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr,
                                      uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rs));
}


// One operand's copies of one K step for one wave: NCH 16-byte copies per
// lane into the wave's NCH * 64 consecutive LDS slots.  M0 holds the LDS
// address of the wave's first slot; copy i adds i KiB through the
// instruction offset, which the direct-to-LDS load applies to both the
// global and the LDS address, so one M0 value serves every copy.  Written
// as inline assembly so that the compiler does not treat the copies as
// pending LDS stores that every later LDS read must wait for: the kernel
// orders copies and reads itself with s_waitcnt vmcnt and barriers.  The
// s_nop covers the wait state between an M0 write and a direct-to-LDS load.
// The compiler's hazard checks do not look inside the assembly: a scalar
// operand (descriptor word) written by a vector instruction -- a spilled
// scalar restored with v_readlane, a v_readfirstlane -- would need five wait
// states before the load reads it.  The kernels keep their descriptors in
// scalar arithmetic and spill no scalars; a build-time test checks the
// compiled code for both.
template <int NCH>
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t rs, uint32_t m0v,
                                          const uint32_t (&v)[NCH]) {
  static_assert(NCH >= 1 && NCH <= 4, "1 to 4 copies of 1 KiB per wave");
  if constexpr (NCH == 1)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "{m0}"(m0v), "v"(v[0]), "s"(rs));
  else if constexpr (NCH == 2)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
                 :: "{m0}"(m0v), "v"(v[0]), "v"(v[1]), "s"(rs));
  else if constexpr (NCH == 3)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %4, 0 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %4, 0 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %4, 0 offen offset:2048 lds"
                 :: "{m0}"(m0v), "v"(v[0]), "v"(v[1]), "v"(v[2]), "s"(rs));
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
                 :: "{m0}"(m0v), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(rs));
}

// One operand's copies and fragment reads.  R: tile rows (m for A, n for B);
// KC: k-contiguous storage.
//
// Copy i of lane l of wave w fills LDS slot (w * NCH + i) * 64 + l; the
// chunk it fetches is the one the slot holds under the swizzle.  The buffer
// descriptor of a K step is based BIAS = (NCH - 1) KiB before the step's
// first byte and each copy's offset register holds its chunk's offset plus
// BIAS minus the instruction offset i KiB: never negative, and the address
// the copy reads and the offset the record check sees are the chunk's own
// (plus BIAS on both sides of the check).  The descriptor advances by one
// K step per step: the base moves on and the record count shrinks, both in
// loop-carried scalar registers.
template <class TL, int R, bool KC>
struct DmaOperand {
  static constexpr int CHUNKS = R * 32 * 2 / 16;         // 16-byte chunks per stage
  static constexpr int NCH = CHUNKS / TL::THREADS;       // per thread per stage
  static constexpr int BYTES = R * 64;                   // one stage of this operand
  static constexpr uint32_t BIAS = (NCH - 1) * 1024;
  static_assert(CHUNKS % TL::THREADS == 0, "whole copy iterations");
  static_assert(KC || R >= 128, "the rows-contiguous swizzle needs 16 chunks per k row");
  // power-of-two R: the slot maps are GF(2)-linear bijections and their
  // derived inverses undo them exactly; any R: the inverses are exact
  static_assert(!is_pow2(R) || TL::template slot_maps_linear<R>(), "linear, bijective slot maps");
  static_assert(!is_pow2(R) ||
                    (gf2::equal(gf2::compose(TL::template kc_slot_inv<R>,
                                             TL::template kc_slot_lin<R>()),
                                gf2::identity(ilog2(R) + 2)) &&
                     gf2::equal(gf2::compose(TL::template mn_slot_inv<R>,
                                             TL::template mn_slot_lin<R>()),
                                gf2::identity(ilog2(R / 8) + 5))),
                "derived inverse slot maps");
  static_assert(TL::template slot_inverses_exact<R>(), "inverse slot maps");
  // k-contiguous: a lane's copies sit 64 slots (16 rows) apart and the
  // swizzle only reads row bits 1-3, so all of them carry the same k chunk
  static constexpr bool same_chunk_per_lane() {
    for (int s = 0; s + 64 < 4 * R; ++s)
      if (TL::template kc_slot_g<R>(s) != TL::template kc_slot_g<R>(s + 64)) return false;
    return true;
  }
  static_assert(!KC || same_chunk_per_lane(), "one k chunk per lane");

  const char* cur;       // descriptor base of the next step's copies
  uint32_t rem;          // its record count while the step is live
  uint32_t step_bytes;   // bytes per K step of 32
  uint32_t voff[NCH];    // per copy: chunk offset + BIAS - i KiB
  uint32_t tail_drop;    // k-contiguous: 2^31 where the lane's chunk lies past K
                         // on the last, partial K step, else 0

  __device__ __forceinline__ void init(const uint16_t* X, int64_t ld, int64_t ext, int row0,
                                       int wave, int lane, int K) {
    cur = reinterpret_cast<const char*>(X) - BIAS;
    rem = (uint32_t)ext + BIAS;
    int kchunk = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int s = (wave * NCH + i) * 64 + lane;  // LDS slot this copy fills
      uint32_t off;
      if (KC) {
        const int r = TL::template kc_slot_row<R>(s), g = TL::template kc_slot_g<R>(s);
        off = (uint32_t)(((int64_t)(row0 + r) * ld + 8 * g) * 2);
        kchunk = 8 * g;
      } else {
        const int k = TL::template mn_slot_k<R>(s), c = TL::template mn_slot_c<R>(s);
        off = (uint32_t)(((int64_t)k * ld + row0 + 8 * c) * 2);
      }
      voff[i] = off + BIAS - 1024u * i;
    }
    step_bytes = (uint32_t)(KC ? 64 : 64 * ld);
    const int nk = (K + 31) / 32;
    tail_drop = (KC && (K & 31) && (nk - 1) * 32 + kchunk >= K) ? 0x80000000u : 0u;
  }

  // Copies of K step `step` of nk into the LDS region at `m0v` (the wave's
  // first slot); then the descriptor moves to the next step.  CHECKED:
  // steps at or after nk (issued ahead of the last step by the pipeline) get
  // zero records, so every copy reads zero and fetches nothing, and on the
  // last, partial step of a k-contiguous operand the chunks at k >= K are
  // pushed out of range (offset + 2^31 exceeds every record count).
  // Unchecked (the caller knows step < nk - 1): neither test, which saves
  // the main loop six vector and about as many scalar instructions per step.
  template <bool CHECKED>
  __device__ __forceinline__ void issue(int step, int nk, uint32_t m0v) {
    uint32_t v[NCH];
    int records = (int)rem;
    if constexpr (CHECKED) {
      records = step < nk ? (int)rem : 0;
      const uint32_t drop = (KC && step == nk - 1) ? tail_drop : 0u;
#pragma unroll
      for (int i = 0; i < NCH; ++i) v[i] = KC ? (voff[i] | drop) : voff[i];
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) v[i] = voff[i];
    }
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)cur, (short)0, records, kBufferFormat);
    dma_block<NCH>(rs, m0v, v);
    cur += step_bytes;
    rem -= step_bytes;
  }
};

// Fused epilogue of a pipelined tile, restaged through LDS.  The tile is
// written in two passes of half its fragment rows: each wave stores its raw
// fp32 accumulators of the pass into an LDS staging array -- rows of BN
// floats, the 16-byte column group g of staged row r at position g XOR
// (r mod 16), so that the 16 rows one fragment store touches fall on
// distinct banks while every aligned run of 16 groups (256 bytes) stays in
// its place, whatever the row width; then every thread takes four
// consecutive columns of successive rows,
// multiplies by the row scale, adds the bias it read once for those columns,
// applies ReLU, adds the residual, rounds once to the output type OT and
// stores one vector -- a wave covers 64 consecutive runs of a row ("My
// Triton From Scratch, Part 16: Register Tiles", sections "Masks and stores"
// and "Broadcasts cannot be treated as full register tiles": per-element
// masks, bias held once per owned column).
//
// MODE, chosen once per tile: EPI_FAST when vector runs are allowed and
// every run of four columns lies wholly inside or wholly outside C (the
// tile's columns are inside C, or N is a multiple of 4), EPI_FAST_RES with a
// residual; either with EPI_SCALED added when there is a row scale, and
// EPI_RELU with ReLU; else EPI_MASKED.
// The fast modes have no branch in the store phase: the residual rows (and
// row scales) of a pass are loaded before its staging writes, and the LDS
// reads of a batch of rows are all issued before the first of their stores.
// They reach C, the residual and the row scale through buffer descriptors
// based at the tile's first row, whose record counts end at row M: a store
// to a row past M is dropped and a load from one reads zero, so a tile whose
// last rows lie past M needs no test per element.  Columns past N are
// handled the same way: the thread's offset for such a run is pushed past
// 2^31, beyond every record count.  An access's byte offset is a part
// common to the workgroup (scalar registers) plus one offset per thread and
// column panel, the same for every item.
// EPI_MASKED masks and stores every element on its own.
enum { EPI_MASKED = 0, EPI_FAST = 1, EPI_FAST_RES = 2, EPI_SCALED = 4, EPI_RELU = 8 };

// Largest leading dimension (elements) of C and of the residual that the fast
// modes take: every byte offset into a tile of at most 256 rows of 4-byte
// elements then stays below 2^31 (and with 2^31 added for a run past N,
// below 2^32).
constexpr int64_t kEpiFastMaxLd = int64_t(1) << 21;

// The store phase works on items: one item is a row of one column panel,
// PANEL columns wide (the whole tile row when BN is a power of two, else 64
// columns), handled by PANEL / 4 threads that own 4 consecutive columns
// each.  Iteration `it` of a thread covers panel it % PANELS of staged row
// (it / PANELS) * ROWS_PER_STEP + t / T_PER_ROW: a thread walks the panels
// of one row before moving on, so the panel of every iteration -- and the
// bias it needs -- is known at compile time.
template <class TL>
struct EpiShape {
  static constexpr int BN = TL::BN, FM = TL::FM, FN = TL::FN;
  static constexpr int PANEL = is_pow2(BN) ? BN : 64;
  static constexpr int PANELS = BN / PANEL;
  static constexpr int COLS_PER_T = 4;
  static constexpr int T_PER_ROW = PANEL / COLS_PER_T;
  static constexpr int ROWS_PER_STEP = TL::THREADS / T_PER_ROW;
  static constexpr int HALF_ROWS = TL::BM / 2;        // staged rows per pass
  static constexpr int ITERS = HALF_ROWS / ROWS_PER_STEP * PANELS;
  static_assert(BN % PANEL == 0 && TL::THREADS % T_PER_ROW == 0 &&
                    HALF_ROWS % ROWS_PER_STEP == 0,
                "whole rows per step");
  static_assert(TL::BM <= 256 && TL::BM * 4 * kEpiFastMaxLd <= (int64_t(1) << 31),
                "byte offsets into the tile stay below 2^31");

  // Staging of the two passes.  Pass 0 takes the upper half of every wave's
  // rows (fragment rows fm < FM/2), pass 1 the lower half; a staged row
  // holds one tile row.  HW rows of each wave row block per pass.
  static constexpr int HW = TL::WTM / 2;
  TRT_HD static int pass_of(int row) { return (row % TL::WTM) / HW; }
  TRT_HD static int staged_row(int row) { return (row / TL::WTM) * HW + row % HW; }
  TRT_HD static int tile_row(int pass, int prow) {
    return (prow / HW) * TL::WTM + HW * pass + prow % HW;
  }
  // Tile row of item `it` of a pass for the threads of the first row of an
  // item (t < T_PER_ROW); thread t takes the row t / T_PER_ROW below it
  // (ROWS_PER_STEP divides HW, so an item's rows stay in one half of a wave
  // row block, where tile_row is a shift).
  static_assert(HW % ROWS_PER_STEP == 0, "an item's rows stay in one half block");
  TRT_HD static int item_row(int pass, int it) {
    return tile_row(pass, (it / PANELS) * ROWS_PER_STEP);
  }

  // The staging writes the accumulators where the layout module's ownership
  // map puts them: for every (register run, lane, wave), the run of four
  // registers 4*(fm*FN + fn) .. +3 is four consecutive columns of one row
  // (starting at a multiple of 4: one 16-byte LDS write), the row is staged
  // in the pass of its fragment row, and its staged row lies in the pass's
  // range and maps back to it.  With the ownership map exactly once (checked
  // where the tile is registered) every tile element is staged once per
  // launch and stored from the row tile_row() gives back.
  static constexpr bool staging_matches_owner() {
    for (int w = 0; w < TL::WAVES; ++w)
      for (int l = 0; l < 64; ++l)
        for (int fm = 0; fm < FM; ++fm)
          for (int fn = 0; fn < FN; ++fn) {
            const int reg = TL::FRAG_REGS * (fm * FN + fn);
            const int row = TL::owner_row(reg, l, w), col = TL::owner_col(reg, l, w);
            if (col % 4 != 0) return false;
            for (int r = 1; r < 4; ++r)
              if (TL::owner_row(reg + r, l, w) != row || TL::owner_col(reg + r, l, w) != col + r)
                return false;
            const int pass = fm < FM / 2 ? 0 : 1;
            const int prow = staged_row(row);
            if (pass_of(row) != pass || prow < 0 || prow >= HALF_ROWS ||
                tile_row(pass, prow) != row)
              return false;
          }
    return true;
  }
};

template <class TL, int OT, int MODE_>
__device__ __forceinline__ void epilogue_passes(const GemmArgs& p,
                                                const f32x4 (&acc)[TL::FM][TL::FN],
                                                float* stage, int m0, int n0, int t,
                                                const float (&bias)[EpiShape<TL>::PANELS][4]) {
  using O = Out<OT>;
  using ES = EpiShape<TL>;
  constexpr int MODE = MODE_ & 3;                      // EPI_MASKED / EPI_FAST / EPI_FAST_RES
  constexpr bool SCALED = (MODE_ & EPI_SCALED) != 0;   // fast modes: row scale present
  constexpr bool RELU = (MODE_ & EPI_RELU) != 0;       // fast modes: ReLU
  constexpr int BN = TL::BN, FM = TL::FM, FN = TL::FN;
  constexpr int PITCH = BN;                           // floats per staged row
  static_assert(BN % 64 == 0, "whole runs of 16 column groups per staged row");
  // float index of the 4-aligned column c of staged row r
  auto sidx = [](int r, int c) { return r * PITCH + ((((c >> 2) ^ (r & 15))) << 2); };
  constexpr int PANELS = ES::PANELS, T_PER_ROW = ES::T_PER_ROW;
  constexpr int ITERS = ES::ITERS;
  // items read ahead of their stores: 8 for 16-bit outputs, 4 for binary32
  // (whose residual ring already holds 64 registers; with 8 the compiler
  // spills, 4 % slower on the rowscale workload)
  constexpr int BATCH = O::BYTES == 2 ? 8 : 4;
  static_assert(FM % 2 == 0 && TL::WM == 2, "two passes over the wave rows");
  static_assert(ITERS % BATCH == 0, "whole batches");
  static_assert(TL::FRAG_REGS == 4 && ES::staging_matches_owner(),
                "the staging follows the tile's ownership map");
  const int lane = t & 63, wave = t >> 6;
  const int tcol = ES::COLS_PER_T * (t % T_PER_ROW);  // this thread's 4 columns in a panel
  const bool relu = p.relu != 0;
  const bool scaled = p.scale != nullptr;
  // iteration it -> staged row, panel, tile column (the panel is a
  // compile-time constant once the loops are unrolled)
  auto prow_of = [&](int it) { return (it / PANELS) * ES::ROWS_PER_STEP + t / T_PER_ROW; };
  auto col_of = [&](int it) { return (it % PANELS) * ES::PANEL + tcol; };
  auto bias_of = [&](int it, int e) { return bias[it % PANELS][e]; };
  // Residuals and row scales travel in a ring of RING items per thread, at
  // most 64 registers of residual (the whole pass for 16-bit outputs, up to
  // 16 items for binary32).  Item `it` is loaded when its slot frees, i.e.
  // right after item it - RING was used, so each load has at least one batch
  // of stores ahead of it; the first RING items are loaded before the
  // staging writes.  For 16-bit outputs (EARLY) the second pass's residual
  // is loaded right after the first pass's staging writes, when half the
  // accumulators are free, so that its latency passes under the first
  // pass's stores (+0.6 % on the epilogue workload).
  constexpr int RING = O::BYTES == 2 ? ITERS : (ITERS < 16 ? ITERS : 16);
  static_assert(RING >= BATCH, "a batch fits the ring");
  auto row_of = [&](int pass, int it) { return m0 + ES::tile_row(pass, prow_of(it)); };
  // Fast modes: the byte offset of item `it` of a pass from the tile's
  // corner in a matrix with leading dimension ld is a part common to the
  // workgroup plus the thread's offset (row t / T_PER_ROW of the item,
  // column tcol).  The common part is walked from item to item in the order
  // the items are accessed; the empty asm keeps the compiler from computing
  // every item's offset ahead, which would take more scalar registers than
  // there are.  Descriptors: based at the tile's first row (and column),
  // records up to row min(M, m0 + BM).
  const int trow = t / T_PER_ROW;
  const int rows = p.M - m0 < TL::BM ? p.M - m0 : TL::BM;
  auto desc = [&](const void* base, int64_t ld, int64_t col) {
    // integer arithmetic: base is null for an absent operand (the descriptor is then unused)
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)((uintptr_t)base + (uintptr_t)(((int64_t)m0 * ld + col) * O::BYTES)), (short)0,
        (int)((uint32_t)rows * (uint32_t)ld * O::BYTES), kBufferFormat);
  };
  auto first = [&](int64_t ld, int pass) { return (uint32_t)(ES::item_row(pass, 0) * ld) * O::BYTES; };
  auto advance = [&](uint32_t& q, int64_t ld, int pass, int it) {  // item it -> it + 1
    const int dr = ES::item_row(pass, it + 1) - ES::item_row(pass, it);
    const int dc = ((it + 1) % PANELS - it % PANELS) * ES::PANEL;
    q += (uint32_t)(dr * ld + dc) * O::BYTES;
    asm volatile("" : "+s"(q));
  };
  // per column panel: the thread's run of four columns inside C, or not
  uint32_t c_off[PANELS], r_off[PANELS];
#pragma unroll
  for (int q = 0; q < PANELS; ++q) {
    const uint32_t out = n0 + q * ES::PANEL + tcol < p.N ? 0u : 0x80000000u;
    c_off[q] = (uint32_t)(trow * p.ldc + tcol) * O::BYTES | out;
    r_off[q] = (uint32_t)(trow * p.ldr + tcol) * O::BYTES | out;
  }
  const uint32_t s_off = (uint32_t)trow * O::BYTES;
  constexpr bool EARLY = MODE == EPI_FAST_RES && O::BYTES == 2 && RING == ITERS;
  typename O::Vec rr_all[EARLY ? 2 : 1][MODE == EPI_FAST_RES ? RING : 1];
  const auto rdesc = desc(p.R, p.ldr, n0), sdesc = desc(p.scale, 1, 0), cdesc = desc(p.C, p.ldc, n0);
  auto fetch_res = [&](int ps) {
    uint32_t q = first(p.ldr, ps);
#pragma unroll
    for (int it = 0; it < RING; ++it) {
      rr_all[ps][it] = O::ld4_buf(rdesc, q + r_off[it % PANELS]);
      advance(q, p.ldr, ps, it);
    }
  };
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    auto& rr = rr_all[EARLY ? pass : 0];
    if constexpr (EARLY) if (pass == 0) fetch_res(0);
    float sc[SCALED ? RING : 1];
    // residual and row-scale items are fetched in ascending order
    uint32_t rq = first(p.ldr, pass), sq = first(1, pass);
    auto fetch = [&](int it) {
      if constexpr (MODE == EPI_FAST_RES && !EARLY) {
        rr[it % RING] = O::ld4_buf(rdesc, rq + r_off[it % PANELS]);
        advance(rq, p.ldr, pass, it);
      }
      if constexpr (SCALED) {
        sc[it % RING] = O::ld_buf(sdesc, sq + s_off);
        sq += (uint32_t)(ES::item_row(pass, it + 1) - ES::item_row(pass, it)) * O::BYTES;
        asm volatile("" : "+s"(sq));
      }
    };
#pragma unroll
    for (int it = 0; it < RING; ++it) fetch(it);
    // the pass's fragment rows fm = (FM/2)*pass + f: each run of four
    // accumulator registers goes to the (row, column) the ownership map
    // gives it, the row staged at staged_row(row)
#pragma unroll
    for (int f = 0; f < FM / 2; ++f) {
      const int fm = (FM / 2) * pass + f;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int reg = TL::FRAG_REGS * (fm * FN + fn);
        const int prow = ES::staged_row(TL::owner_row(reg, lane, wave));
        const int c = TL::owner_col(reg, lane, wave);
        *reinterpret_cast<f32x4*>(stage + sidx(prow, c)) = acc[fm][fn];
      }
    }
    if constexpr (EARLY) if (pass == 0) fetch_res(1);
    __syncthreads();
    if constexpr (MODE != EPI_MASKED) {
      uint32_t cq = first(p.ldc, pass);   // C items are stored in ascending order
#pragma unroll
      for (int b0 = 0; b0 < ITERS; b0 += BATCH) {
        f32x4 v[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          v[i] = *reinterpret_cast<const f32x4*>(stage + sidx(prow_of(b0 + i), col_of(b0 + i)));
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
          const int it = b0 + i;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // an absent bias is -0, an exact identity (-0 included), so no
            // select is needed
            y[e] = (SCALED ? v[i][e] * sc[it % RING] : v[i][e]) + bias_of(it, e);
            if constexpr (RELU) y[e] = y[e] > 0.f ? y[e] : 0.f;
            if constexpr (MODE == EPI_FAST_RES) y[e] += O::elem(rr[it % RING], e);
          }
          O::st4_buf(cdesc, cq + c_off[it % PANELS], O::pack(y));
          advance(cq, p.ldc, pass, it);
        }
        // the batch's slots are free: fetch the items RING further on
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          if (b0 + i + RING < ITERS) fetch(b0 + i + RING);
      }
    } else {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int m = row_of(pass, it);
        const int n = n0 + col_of(it);
        if (m >= p.M) continue;
        const bool vec = p.epi_vec && n + 4 <= p.N;
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(stage + sidx(prow_of(it), col_of(it)));
        float y[4] = {a4[0], a4[1], a4[2], a4[3]};
        if (scaled) {
          const float s = O::ld(p.scale, m);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] *= s;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] += bias_of(it, e);
        if (relu) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = y[e] > 0.f ? y[e] : 0.f;
        }
        if (p.R) {
          const int64_t r0 = (int64_t)m * p.ldr + n;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) y[e] += O::ld(p.R, r0 + e);
        }
        const int64_t c0 = (int64_t)m * p.ldc + n;
        if (vec) {
          O::st4(p.C, c0, O::pack(y));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) O::st(p.C, c0 + e, y[e]);
        }
      }
    }
    __syncthreads();
  }
}

template <class TL, int OT>
__device__ __forceinline__ void epilogue_lds(const GemmArgs& p, const f32x4 (&acc)[TL::FM][TL::FN],
                                             float* stage, int m0, int n0, int t) {
  using O = Out<OT>;
  using ES = EpiShape<TL>;
  // the bias of this thread's 4 columns in every panel; -0 where there is
  // none: x + (-0) == x for every x, -0 included
  float bias[ES::PANELS][4];
#pragma unroll
  for (int q = 0; q < ES::PANELS; ++q) {
    const int n = n0 + q * ES::PANEL + ES::COLS_PER_T * (t % ES::T_PER_ROW);
    const bool vec = p.epi_vec && n + 4 <= p.N;
#pragma unroll
    for (int e = 0; e < 4; ++e) bias[q][e] = -0.f;
    if (p.bias) {
      if (vec) {
        const auto bb = O::ld4(p.bias, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[q][e] = O::elem(bb, e);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) bias[q][e] = O::ld(p.bias, n + e);
      }
    }
  }
  // a residual whose rows overlap (ldr < N) has real columns past its
  // record count: it takes the masked phase
  const bool fast = p.epi_vec && (n0 + TL::BN <= p.N || p.N % 4 == 0) &&
                    p.ldc < kEpiFastMaxLd && (!p.R || (p.ldr >= p.N && p.ldr < kEpiFastMaxLd));
  auto run = [&]<int MODE>() { epilogue_passes<TL, OT, MODE>(p, acc, stage, m0, n0, t, bias); };
  auto fast_relu = [&]<int MODE>() {
    if (p.relu) run.template operator()<MODE | EPI_RELU>();
    else run.template operator()<MODE>();
  };
  if (!fast)
    run.template operator()<EPI_MASKED>();
  else if (p.scale)
    if (p.R) fast_relu.template operator()<EPI_FAST_RES | EPI_SCALED>();
    else fast_relu.template operator()<EPI_FAST | EPI_SCALED>();
  else if (p.R)
    fast_relu.template operator()<EPI_FAST_RES>();
  else
    fast_relu.template operator()<EPI_FAST>();
}

// Fragment addressing for 16-row fragments.  Lane group g = lane/16
// supplies k chunk kchunk(g) = (0, 3, 1, 2)[g] (8 consecutive k); any
// order common to both operands gives the same sum, and this one keeps
// the 16-byte reads free of bank conflicts: groups g and g+1 read the same
// 16 rows, and measured on gfx950 only chunk pairs differing in both bits
// (0/3, 1/2) cost no extra LDS cycles, whatever the swizzle.
// k-contiguous: one base, the swizzle repeats every 16 rows, so fragment f
// sits 1024 bytes further.  rows-contiguous: lane j of group g reads 4 rows
// at k = 8*kchunk(g) + j/4, chunk (j%4)/2, half j%2 (the transposing read
// hands lane i row i of the 4 k), and the next 4 k at +8R bytes; one base
// per fragment.
__device__ __forceinline__ int frag_kchunk(int g) { return (g & 1) ? 3 - (g >> 1) : (g >> 1); }

template <class TL, int R, bool KC, int F>
struct FragReader {
  int addr[KC ? 1 : F];

  __device__ __forceinline__ void init(int rbase, int lane, int region) {
    const int g = frag_kchunk(lane >> 4);
    if (KC) {
      addr[0] = region + 16 * TL::kc_slot(rbase + (lane & 15), g);
    } else {
      const int j = lane & 15;
      const int k = 8 * g + (j >> 2);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int c = (rbase + 16 * f) / 8 + ((j & 3) >> 1);
        addr[f] = region + 16 * (k * (R / 8) + (c ^ TL::template mn_swz<R>(k))) + 8 * (j & 1);
      }
    }
  }

  __device__ __forceinline__ u32x4 read(TRT_LDS char* st, int f) const {
    if (KC) return *(TRT_LDS u32x4*)(st + addr[0] + 1024 * f);
    TRT_LDS char* p = st + addr[f];
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TRT_LDS i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TRT_LDS i16x4*)(p + 8 * R));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
};

// Per K step one block of FM*FN products on one set of operand registers:
// the first half (fragment rows 0..FM/2-1 against every column, column by
// column) with this thread's copies of step kt+3 and the reads of the step's
// own rows FM/2..FM-1 spread through it; then the wait for those reads and
// for step kt+1's copies, and the barrier; then the second half (rows
// FM/2..FM-1, column by column) with the next stage's rows 0..FM/2-1 and
// columns read into the registers as they die (each column right after its
// last product).
template <class TL, int DT, bool A_KC, bool B_KC, int NS = 4>
__global__ __launch_bounds__(TL::THREADS, 1) void gemm_dma_kernel(GemmArgs p) {
  static_assert(TL::BK == 32 && TL::MF == 16, "32-wide K steps of 16x16x32 fragments");
  static_assert(NS >= 3, "copies at least two steps ahead");
  constexpr int BM = TL::BM, BN = TL::BN, FM = TL::FM, FN = TL::FN;
  constexpr int HM = FM / 2, HALF = HM * FN;
  using OpA = DmaOperand<TL, BM, A_KC>;
  using OpB = DmaOperand<TL, BN, B_KC>;
  constexpr int STAGE = OpA::BYTES + OpB::BYTES;
  constexpr int LOADS = OpA::NCH + OpB::NCH;
  constexpr int EPI_BYTES = (BM / 2) * BN * 4;
  constexpr int LDS_BYTES = NS * STAGE > EPI_BYTES ? NS * STAGE : EPI_BYTES;
  static_assert(FM % 2 == 0 && HALF >= 2, "copies fit the first half");
  __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
  TRT_LDS char* lds = (TRT_LDS char*)lds_raw;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int tm, tn;
  tile_of<8>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  OpA a;
  OpB b;
  a.init(p.A, p.lda, p.a_bytes, m0, wave, lane, p.K);
  b.init(p.B, p.ldb, p.b_bytes, n0, wave, lane, p.K);

  const int nk = (p.K + 31) / 32;
  // LDS address of this wave's first copy slot in each operand region of
  // stage 0 (wave-uniform)
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const uint32_t m0a = __builtin_amdgcn_readfirstlane(lds_base + wave * OpA::NCH * 1024);
  const uint32_t m0b =
      __builtin_amdgcn_readfirstlane(lds_base + OpA::BYTES + wave * OpB::NCH * 1024);

  // fragment reads start at the wave's first tile row / column: where the
  // ownership map places register 0 of lane 0
  FragReader<TL, BM, A_KC, FM> ra;
  FragReader<TL, BN, B_KC, FN> rb;
  ra.init(TL::owner_row(0, 0, wave), lane, 0);
  rb.init(TL::owner_col(0, 0, wave), lane, OpA::BYTES);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 fa[FM], fb[FN];

  // Fragment f of a step in the order the schedule reads it: the first HM
  // A fragments, then the B fragments, then the other A fragments.
  auto read_frag = [&](TRT_LDS char* st, int f) __attribute__((always_inline)) {
    if (f < HM) fa[f] = ra.read(st, f);
    else if (f < HM + FN) fb[f - HM] = rb.read(st, f - HM);
    else fa[f - FN] = ra.read(st, f - FN);
  };

  // Stage of K step s: (s - r) mod NS, r = nk mod NS.  The first r steps
  // run with run-time stage offsets; the main loop then starts at step r
  // and runs whole rounds of NS steps, unrolled, in which every stage
  // offset -- of the copies issued in step kt (step kt+NS-1) and of the
  // fragments read in it (step kt+1) -- is a constant: the LDS reads take it
  // in their offset field and the copies in their M0 value.
  const int r = nk % NS;
  auto stage_of = [&](int s) { return (uint32_t)((s - r + NS) % NS) * STAGE; };

  // prologue: steps 0..NS-2 in flight, step 0's fragments in registers
#pragma unroll
  for (int step = 0; step < NS - 1; ++step) {
    a.template issue<true>(step, nk, m0a + stage_of(step));
    b.template issue<true>(step, nk, m0b + stage_of(step));
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * LOADS));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // the epilogue's strides in scalar registers before the loop: a scalar
  // load still in flight at the loop's entry would force a full LDS wait
  // (scalar loads complete out of order) at the top of every round
  asm volatile("" ::"s"(p.ldc), "s"(p.ldr));
  // in the order the steps read them, so that the wait counts agree (the
  // lower A rows are read by each step itself, in its first half)
#pragma unroll
  for (int f = 0; f < HM + FN; ++f) read_frag(lds + stage_of(0), f);

  // One K step kt: the copies of step kt+NS-1 go to stage offset `cst`, the
  // fragments of step kt+1 come from `nxt`; CHECKED as in DmaOperand::issue.
  auto step_body = [&]<bool CHECKED>(int kt, uint32_t cst, TRT_LDS char* cur, TRT_LDS char* nxt) __attribute__((always_inline)) {
    const int step = kt + NS - 1;
    // first half, column by column: the column fragment read last in the
    // previous step is needed last; this step's A rows HM..FM-1 read from
    // its own stage after every second product (they are used after the
    // barrier); A's copies halfway through, B's two products before the end
    // (measured 1 % faster than copies after the first product and halfway,
    // and than three other placements)
#pragma unroll
    for (int q = 0; q < HALF; ++q) {
      const int j = q / HM, i = q % HM;
      acc[i][j] = mfma16<DT>(fb[j], fa[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (q == HALF / 2) a.template issue<CHECKED>(step, nk, m0a + cst);
      if (q == HALF - 2) b.template issue<CHECKED>(step, nk, m0b + cst);
      if (q % 2 == 1 && q / 2 < FM - HM) read_frag(cur, HM + FN + q / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every read of the stage that the next step's copies overwrite was
    // issued before this point: complete the reads, and step kt+1's copies,
    // before the barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * LOADS));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // second half: the next step's fragments into the registers as they die
    // -- rows 0..HM-1 first, each column after its last product (rows
    // HM..FM-1 of the next step are read in its own first half, once this
    // step's second half has used them)
#pragma unroll
    for (int q = 0; q < HALF; ++q) {
      const int j = q / HM, i = HM + q % HM;
      acc[i][j] = mfma16<DT>(fb[j], fa[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (q < HM) read_frag(nxt, q);
      if (q % HM == HM - 1) read_frag(nxt, HM + j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int kt = 0; kt < r; ++kt)
    step_body.template operator()<true>(kt, stage_of(kt + NS - 1), lds + stage_of(kt),
                                        lds + stage_of(kt + 1));
  // Whole rounds of NS steps from step r: every round but the last copies
  // live steps before the last one only (a round from kt copies steps
  // kt+NS-1 .. kt+2NS-2 <= nk-2), so it runs unchecked; the last round
  // copies the last step and the steps past the end.
  int kt = r;
  for (; kt < nk - NS; kt += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      step_body.template operator()<false>(kt + u, ((u + NS - 1) % NS) * STAGE, lds + u * STAGE,
                                           lds + ((u + 1) % NS) * STAGE);
  }
  if (kt < nk) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      step_body.template operator()<true>(kt + u, ((u + NS - 1) % NS) * STAGE, lds + u * STAGE,
                                          lds + ((u + 1) % NS) * STAGE);
  }
  // drain the copies issued past the end (zero records: they fetch nothing)
  // and all LDS reads before the staging area reuses the stages
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  __syncthreads();

  with_out_type(p.out_dt, [&]<int OT>() {
    epilogue_lds<TL, OT>(p, acc, reinterpret_cast<float*>(lds_raw), m0, n0, t);
  });
}

}  // namespace trt
