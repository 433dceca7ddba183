// layout.hpp -- the layout module: who owns, moves and stores which element.
//
// Three shapes are kept apart ("My Triton From Scratch, Part 16: Register
// Tiles", section "Three coordinate spaces"):
//   * the logical tile   [BM, BN]  -- the C elements one workgroup produces;
//   * the thread shape   WM x WN wavefronts of 64 lanes (physical);
//   * the register shape FM x FN fragments x 4 fp32 registers per lane.
//
// Every map is GF(2)-linear in the bits of its inputs ("Triton LinearLayout",
// sections "Linear Layout" and "Basis-vector representation"): a value is
// the XOR of the basis vectors its set input bits select.  The C ownership
// (register, lane, wave) -> (row, col) is stated twice -- as the arithmetic
// the kernel evaluates and as GF(2) bases -- and a compile-time check proves
// the two agree everywhere and that the basis matrix is square with full
// rank, i.e. every output element is owned exactly once ("Triton
// LinearLayout", section "Surjectivity, injectivity, and broadcasts").
//
// Matrix-core fragments, one wave of 64 lanes (AMD's documented register
// layouts of v_mfma_f32_16x16x32_* and v_mfma_f32_32x32x16_*):
//   16x16x32: operand 0 (16 x 32): lane l holds row l%16, k = 8*(l/16) + e;
//             operand 1 (32 x 16): column l%16, the same k rule;
//             result (16 x 16): lane l, register r is row 4*(l/16) + r, col l%16.
//   32x32x16: operand 0 (32 x 16): lane l holds row l%32, k = 8*(l/32) + e;
//             operand 1 (16 x 32): column l%32, the same k rule;
//             result (32 x 32): lane l, register r is row 8*(r/4) + 4*(l/32) + r%4,
//             col l%32.
// The k rule only has to agree between the two operands (the instruction
// sums over k slots).  The kernels feed the B tile (rows = n) to operand 0
// and the A tile (rows = m) to operand 1, so a fragment result is a C^T
// fragment: every run of four consecutive registers of a lane holds four
// consecutive columns of one C row, which the epilogue stores as one 8-byte
// vector.
#pragma once

#include <stdint.h>

#define TRT_HD __host__ __device__ __forceinline__ constexpr

namespace trt {

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }
constexpr bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// One basis vector: the (row, col) image of one input bit.
struct Basis {
  int32_t row, col;
};

// A GF(2)-linear map from NIN input bits to (row, col).
template <int NIN>
struct Gf2Map {
  Basis b[NIN];
  int row_bits, col_bits;

  // XOR of the bases selected by the set bits of x ("Triton LinearLayout",
  // section "LinearLayout::apply").
  constexpr Basis apply(uint32_t x) const {
    Basis out{0, 0};
    for (int i = 0; i < NIN; ++i)
      if ((x >> i) & 1u) {
        out.row ^= b[i].row;
        out.col ^= b[i].col;
      }
    return out;
  }

  // Rank over GF(2) of the matrix whose columns are the bases, by Gaussian
  // elimination on packed (row | col << row_bits) words.
  constexpr int rank() const {
    uint32_t w[NIN] = {};
    for (int i = 0; i < NIN; ++i)
      w[i] = uint32_t(b[i].row) | (uint32_t(b[i].col) << row_bits);
    int r = 0;
    for (int bit = 0; bit < row_bits + col_bits; ++bit) {
      int p = -1;
      for (int i = r; i < NIN; ++i)
        if ((w[i] >> bit) & 1u) { p = i; break; }
      if (p < 0) continue;
      uint32_t t = w[p]; w[p] = w[r]; w[r] = t;
      for (int i = 0; i < NIN; ++i)
        if (i != r && ((w[i] >> bit) & 1u)) w[i] ^= w[r];
      ++r;
    }
    return r;
  }

  // Injective and surjective: a square basis matrix of full rank.
  constexpr bool bijective() const {
    return NIN == row_bits + col_bits && rank() == NIN;
  }
};

// ---------------------------------------------------------------------------
// The layout algebra ("Triton LinearLayout", sections "Combining layouts" and
// "invertAndCompose: derive data movement"), on GF(2)-linear maps of at most
// 32 input bits to at most 32 output bits.  A map is stored by its columns:
// col[i] is the image of input bit i as a packed output word.  The same
// constexpr code derives maps at compile time (the inverse copy maps of the
// pipelined kernel below) and serves the C ABI at run time.
// ---------------------------------------------------------------------------
namespace gf2 {

struct Lin {
  uint32_t col[32];
  int nin, nout;

  constexpr uint32_t apply(uint32_t x) const {
    uint32_t y = 0;
    for (int i = 0; i < nin; ++i)
      if ((x >> i) & 1u) y ^= col[i];
    return y;
  }
  constexpr uint32_t out_mask() const { return nout >= 32 ? 0xFFFFFFFFu : (1u << nout) - 1u; }
};

constexpr Lin zero(int nin, int nout) {
  Lin l{};
  l.nin = nin;
  l.nout = nout;
  return l;
}

constexpr Lin identity(int n) {
  Lin l = zero(n, n);
  for (int i = 0; i < n; ++i) l.col[i] = 1u << i;
  return l;
}

// Echelon basis of a set of words: piv[b] holds a vector whose lowest set bit
// is b (0 when there is none) and comb[b] the combination of the input
// columns that produced it.
struct Echelon {
  uint32_t piv[32], comb[32];
  int rank;

  // Reduce word v (with combination c) by the pivots; returns the rest.
  constexpr uint32_t reduce(uint32_t v, uint32_t& c) const {
    while (v) {
      const int b = __builtin_ctz(v);
      if (!piv[b]) return v;
      v ^= piv[b];
      c ^= comb[b];
    }
    return 0;
  }
};

constexpr Echelon echelon(const Lin& l) {
  Echelon e{};
  for (int i = 0; i < l.nin; ++i) {
    uint32_t c = 1u << i;
    const uint32_t v = e.reduce(l.col[i], c);
    if (v) {
      const int b = __builtin_ctz(v);
      e.piv[b] = v;
      e.comb[b] = c;
      ++e.rank;
    }
  }
  return e;
}

// Rank; injective = rank equals the input bits, surjective = the output bits
// ("Triton LinearLayout", section "Surjectivity, injectivity, and broadcasts").
constexpr int rank(const Lin& l) { return echelon(l).rank; }
constexpr bool injective(const Lin& l) { return rank(l) == l.nin; }
constexpr bool surjective(const Lin& l) { return rank(l) == l.nout; }
constexpr bool bijective(const Lin& l) { return l.nin == l.nout && injective(l); }

// outer o inner: outer applied to every column of inner (outer.nin == inner.nout).
constexpr Lin compose(const Lin& outer, const Lin& inner) {
  Lin l = zero(inner.nin, outer.nout);
  for (int i = 0; i < inner.nin; ++i) l.col[i] = outer.apply(inner.col[i]);
  return l;
}

// Direct sum: the input bits of a then those of b; the output bits of a then
// those of b (a.nin + b.nin <= 32, a.nout + b.nout <= 32).
constexpr Lin product(const Lin& a, const Lin& b) {
  Lin l = zero(a.nin + b.nin, a.nout + b.nout);
  for (int i = 0; i < a.nin; ++i) l.col[i] = a.col[i];
  for (int i = 0; i < b.nin; ++i) l.col[a.nin + i] = b.col[i] << a.nout;
  return l;
}

// Restriction to the input bits set in in_mask and projection onto the
// output bits set in out_mask; kept bits stay in order and are packed.
constexpr Lin sublayout(const Lin& l, uint32_t in_mask, uint32_t out_mask) {
  Lin r = zero(__builtin_popcount(in_mask & (l.nin >= 32 ? 0xFFFFFFFFu : (1u << l.nin) - 1u)),
               __builtin_popcount(out_mask & l.out_mask()));
  int k = 0;
  for (int i = 0; i < l.nin; ++i) {
    if (!((in_mask >> i) & 1u)) continue;
    uint32_t w = 0;
    int o = 0;
    for (int b = 0; b < l.nout; ++b)
      if ((out_mask >> b) & 1u) w |= ((l.col[i] >> b) & 1u) << o++;
    r.col[k++] = w;
  }
  return r;
}

// Given R: X -> T and S: Y -> T (same output bits), a map Q: X -> Y with
// S(Q(x)) == R(x) for every x; false if some value of R is not a value of S.
// S need not be injective (broadcast bits): Q picks, per column of R, the
// solution that uses no column of S dependent on earlier ones.
constexpr bool invert_and_compose(const Lin& R, const Lin& S, Lin& Q) {
  Q = zero(R.nin, S.nin);
  if (R.nout != S.nout) return false;
  const Echelon e = echelon(S);
  for (int i = 0; i < R.nin; ++i) {
    uint32_t c = 0;
    if (e.reduce(R.col[i], c)) return false;
    Q.col[i] = c;
  }
  return true;
}

// Inverse of a bijective map.
constexpr Lin inverse(const Lin& l) {
  Lin q{};
  invert_and_compose(identity(l.nout), l, q);
  return q;
}

constexpr bool equal(const Lin& a, const Lin& b) {
  if (a.nin != b.nin || a.nout != b.nout) return false;
  for (int i = 0; i < a.nin; ++i)
    if (a.col[i] != b.col[i]) return false;
  return true;
}

// The GF(2) map of an integer function f on n input bits, read off its
// values on the unit vectors (meaningful when f is GF(2)-linear; callers
// check that with agrees()).
template <class F>
constexpr Lin from_function(int nin, int nout, F f) {
  Lin l = zero(nin, nout);
  for (int i = 0; i < nin; ++i) l.col[i] = (uint32_t)f(1u << i);
  return l;
}

// apply() with the number of input bits fixed at compile time, for maps
// known at compile time: the loop unrolls and every column folds into an
// immediate, so device code evaluates the map with a few bit operations.
template <int N>
TRT_HD uint32_t apply_n(const Lin& l, uint32_t x) {
  uint32_t y = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) y ^= ((x >> i) & 1u) ? l.col[i] : 0u;
  return y;
}

// Whether f equals the map l on every input.
template <class F>
constexpr bool agrees(const Lin& l, F f) {
  for (uint32_t x = 0; x < (1u << l.nin); ++x)
    if ((uint32_t)f(x) != l.apply(x)) return false;
  return true;
}

}  // namespace gf2

// ---------------------------------------------------------------------------
// A workgroup tile: logical shape, thread shape, register shape.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int BK_, int WM_, int WN_, int MF_ = 16>
struct Tile {
  // logical tile and K step
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  // physical thread shape
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  // per-wave sub-tile, in MF x MF matrix-core fragments (MF = 16 or 32)
  static constexpr int MF = MF_;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / MF, FN = WTN / MF;
  // register shape: accumulator registers per lane
  static constexpr int FRAG_REGS = MF * MF / 64;
  static constexpr bool COPY_MAPS = true;  // has cooperative copy / LDS maps
  static constexpr int REGS = FM * FN * FRAG_REGS;
  // operand tiles in LDS: G chunks of 8 k (16 bytes) per row
  static constexpr int G = BK / 8;
  static constexpr int KSUB = BK / 32;  // matrix-core k steps per K step

  // Power-of-two tiles have a GF(2)-linear ownership map; a tile with a
  // non-power-of-two number of fragments per wave (BN = 192: 3 fragments of
  // 32 columns) has an integer-affine one ("My Triton From Scratch, Part 16:
  // Register Tiles", section "A strided ownership rule").
  static constexpr bool POW2 = is_pow2(BM) && is_pow2(BN) && is_pow2(FM) && is_pow2(FN);
  static_assert(is_pow2(BM) && is_pow2(BK) && (is_pow2(BN) || BN % 64 == 0),
                "power-of-two BM and BK; BN a power of two or a multiple of 64");
  static_assert(is_pow2(WM) && is_pow2(WN), "power-of-two wave grid");
  static_assert(MF == 16 || MF == 32, "16x16 or 32x32 fragments");
  static_assert(WTM >= MF && WTN >= MF && WTM % MF == 0 && WTN % MF == 0,
                "each wave owns whole fragments");
  static_assert(BK >= 32 && BK % 32 == 0 && G <= 8, "K step: 32 or 64");
  static_assert(THREADS <= 1024, "1024 work-items per workgroup at most");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "8x8 transpose blocks");

  // ---- C ownership, as the kernel evaluates it ----------------------------
  // Register index reg = FRAG_REGS*(fm*FN + fn) + r.
  TRT_HD static int owner_row(int reg, int lane, int wave) {
    const int fm = (reg / FRAG_REGS) / FN;
    return (wave / WN) * WTM + MF * fm + (lane & (MF - 1));
  }
  TRT_HD static int owner_col(int reg, int lane, int wave) {
    const int fn = (reg / FRAG_REGS) % FN;
    const int r = reg % FRAG_REGS;
    const int in_frag = MF == 16 ? 4 * (lane >> 4) + r
                                 : 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    return (wave % WN) * WTN + MF * fn + in_frag;
  }

  // Exactly-once ownership by enumeration, for any tile: every (register,
  // lane, wave) lands inside the tile and no element is reached twice; with
  // REGS * 64 * WAVES == BM * BN that also means every element is reached.
  static constexpr bool owner_exactly_once() {
    if (REGS * 64 * WAVES != BM * BN) return false;
    uint64_t seen[BM * BN / 64] = {};
    for (int w = 0; w < WAVES; ++w)
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < REGS; ++r) {
          const int row = owner_row(r, l, w), col = owner_col(r, l, w);
          if (row < 0 || row >= BM || col < 0 || col >= BN) return false;
          const int i = row * BN + col;
          if ((seen[i >> 6] >> (i & 63)) & 1u) return false;
          seen[i >> 6] |= uint64_t(1) << (i & 63);
        }
    return true;
  }

  // ---- the same ownership as GF(2) bases (power-of-two tiles) ---------------
  // Input bits, low to high: register bits, 6 lane bits, wave bits.
  static constexpr int REG_BITS = ilog2(REGS);
  static constexpr int WAVE_BITS = ilog2(WAVES);
  static constexpr int C_IN_BITS = REG_BITS + 6 + WAVE_BITS;

  static constexpr Gf2Map<C_IN_BITS> c_map() {
    Gf2Map<C_IN_BITS> m{};
    m.row_bits = ilog2(BM);
    m.col_bits = ilog2(BN);
    int i = 0;
    m.b[i++] = {0, 1};                                  // r bit 0
    m.b[i++] = {0, 2};                                  // r bit 1
    if (MF == 32) {
      m.b[i++] = {0, 8};                                // r bit 2
      m.b[i++] = {0, 16};                               // r bit 3
    }
    for (int s = 0; s < ilog2(FN); ++s) m.b[i++] = {0, MF << s};   // fn
    for (int s = 0; s < ilog2(FM); ++s) m.b[i++] = {MF << s, 0};   // fm
    for (int s = 0; s < ilog2(MF); ++s) m.b[i++] = {1 << s, 0};    // lane: row
    if (MF == 16) {
      m.b[i++] = {0, 4};                                // lane bits 4-5: col
      m.b[i++] = {0, 8};
    } else {
      m.b[i++] = {0, 4};                                // lane bit 5: col
    }
    for (int s = 0; s < ilog2(WN); ++s) m.b[i++] = {0, WTN << s};  // wave col
    for (int s = 0; s < ilog2(WM); ++s) m.b[i++] = {WTM << s, 0};  // wave row
    return m;
  }

  // Exhaustive agreement of the arithmetic form with the bases.
  static constexpr bool owner_matches_bases() {
    constexpr auto m = c_map();
    for (int w = 0; w < WAVES; ++w)
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < REGS; ++r) {
          const uint32_t x = uint32_t(r) | (uint32_t(l) << REG_BITS) |
                             (uint32_t(w) << (REG_BITS + 6));
          const Basis v = m.apply(x);
          if (v.row != owner_row(r, l, w) || v.col != owner_col(r, l, w)) return false;
        }
    return true;
  }

  static_assert(!POW2 || c_map().bijective(),
                "C ownership must cover every tile element exactly once");
  // The exhaustive owner_matches_bases() check runs once per compiled tile,
  // in the library's tile registry.

  // ---- LDS operand tiles ----------------------------------------------------
  // Chunk (r, g) of a tile with R rows lives in 16-byte slot
  // r*G + (g XOR s(r)),  s(r) = ((r >> (3 - log2 G)) XOR (r >> 3)) mod G.
  // s is linear in the bits of r, so the slot map is a GF(2) bijection.  A
  // fragment read (16 consecutive rows, one g) and a copy write (8 lanes on
  // one row, or 8 lanes on rows 8 apart) both touch distinct 16-byte bank
  // groups within each 128-byte LDS cycle.
  TRT_HD static int lds_swz(int r) {
    return ((r >> (3 - ilog2(G))) ^ (r >> 3)) & (G - 1);
  }
  TRT_HD static int lds_slot(int r, int g) { return r * G + (g ^ lds_swz(r)); }

  // ---- direct-to-LDS operand tiles (K step of 32) ---------------------------
  // The pipelined kernel copies global memory straight into LDS, 16 bytes per
  // lane: the lanes of one wave instruction fill 64 consecutive 16-byte slots,
  // so the swizzle is applied on the global side -- each lane fetches the
  // chunk that belongs in its slot (the inverse maps below).
  //
  // k-contiguous operand, [R rows][4 chunks of 8 k]: chunk (r, g) in slot
  // 4r + (g XOR sk(r)), sk(r) = (r1 XOR r3) | r2 << 1 in the bits of r.  A
  // fragment read (16 consecutive rows, one g, 16 bytes per lane) covers every
  // bank once per 8 rows (128-byte window) and per 16 rows (256-byte window);
  // sk only uses bits 1-3 of r, so fragments 16 rows apart differ by a
  // constant address offset.
  TRT_HD static int kc_swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }
  TRT_HD static int kc_slot(int r, int g) { return 4 * r + (g ^ kc_swz(r)); }
  // The copy side needs the inverse, slot -> (row, chunk).  It is derived
  // with the layout algebra: the slot map as a GF(2) map of (g, r) bits
  // (2 chunk bits low, then the row bits), inverted.
  template <int R>
  static constexpr gf2::Lin kc_slot_lin() {
    constexpr int rb = ilog2(R);
    return gf2::from_function(rb + 2, rb + 2, [](uint32_t x) {
      return (uint32_t)kc_slot((int)(x >> 2), (int)(x & 3));
    });
  }
  template <int R>
  static constexpr gf2::Lin kc_slot_inv = gf2::inverse(kc_slot_lin<R>());
  // (For a non-power-of-two R the slot map is affine, not GF(2)-linear: its
  // inverse is the integer one, row = s / 4, chunk = (s mod 4) XOR sk(row).)
  template <int R>
  TRT_HD static int kc_slot_row(int s) {
    if constexpr (is_pow2(R)) {
      constexpr gf2::Lin inv = kc_slot_inv<R>;
      return (int)(gf2::apply_n<ilog2(R) + 2>(inv, (uint32_t)s) >> 2);
    } else {
      return s >> 2;
    }
  }
  template <int R>
  TRT_HD static int kc_slot_g(int s) {
    if constexpr (is_pow2(R)) {
      constexpr gf2::Lin inv = kc_slot_inv<R>;
      return (int)(gf2::apply_n<ilog2(R) + 2>(inv, (uint32_t)s) & 3u);
    } else {
      return (s & 3) ^ kc_swz(s >> 2);
    }
  }
  // rows-contiguous operand, [32 k rows][R/8 chunks of 8 rows]: chunk (k, c)
  // in slot k*(R/8) + (c XOR sm(k)), sm(k) = 6*k0 XOR 12*k1 XOR 2*k3 in the
  // bits of k.  A transposing fragment read covers 4 consecutive k rows, 32
  // bytes (two chunks) of each per 16 lanes; the 32 lanes served together
  // read two such groups 8 k rows apart (k = 8g + 0..3 for lane group g).
  // k0 and k1 send the four rows of a group to distinct bank groups, and k3
  // moves the second group off the first one's.
  // With 24 chunks per k row (R = 192) the XOR has to stay inside aligned
  // groups of 8 chunks: sm(k) = 6*k0 XOR 4*k1 XOR 2*k3, with the same
  // effect (checked for both widths by enumerating every read's banks).
  template <int R>
  TRT_HD static int mn_swz(int k) {
    return ((R / 8) % 16 == 0 ? (((k & 1) ? 6 : 0) ^ ((k & 2) ? 12 : 0))
                              : (((k & 1) ? 6 : 0) ^ ((k & 2) ? 4 : 0))) ^
           ((k & 8) ? 2 : 0);
  }
  template <int R>
  TRT_HD static int mn_slot(int k, int c) { return k * (R / 8) + (c ^ mn_swz<R>(k)); }
  // The inverse, slot -> (k, chunk), derived like kc_slot_inv: the slot map
  // as a GF(2) map of (c, k) bits (chunk bits low, then 5 k bits), inverted.
  template <int R>
  static constexpr gf2::Lin mn_slot_lin() {
    constexpr int cb = ilog2(R / 8);
    return gf2::from_function(cb + 5, cb + 5, [](uint32_t x) {
      return (uint32_t)mn_slot<R>((int)(x >> cb), (int)(x & ((1u << cb) - 1u)));
    });
  }
  template <int R>
  static constexpr gf2::Lin mn_slot_inv = gf2::inverse(mn_slot_lin<R>());
  template <int R>
  TRT_HD static int mn_slot_k(int s) {
    if constexpr (is_pow2(R)) {
      constexpr gf2::Lin inv = mn_slot_inv<R>;
      return (int)(gf2::apply_n<ilog2(R / 8) + 5>(inv, (uint32_t)s) >> ilog2(R / 8));
    } else {
      return s / (R / 8);
    }
  }
  template <int R>
  TRT_HD static int mn_slot_c(int s) {
    if constexpr (is_pow2(R)) {
      constexpr gf2::Lin inv = mn_slot_inv<R>;
      return (int)(gf2::apply_n<ilog2(R / 8) + 5>(inv, (uint32_t)s) & ((1u << ilog2(R / 8)) - 1u));
    } else {
      return (s % (R / 8)) ^ mn_swz<R>(s / (R / 8));
    }
  }
  // For any R: the inverse maps undo the forward maps on every slot.
  template <int R>
  static constexpr bool slot_inverses_exact() {
    for (int s = 0; s < 4 * R; ++s) {
      if (kc_slot(kc_slot_row<R>(s), kc_slot_g<R>(s)) != s) return false;
      if (mn_slot<R>(mn_slot_k<R>(s), mn_slot_c<R>(s)) != s) return false;
    }
    return true;
  }
  // The derivations hold only if the slot maps are GF(2)-linear bijections:
  // checked on every input.
  template <int R>
  static constexpr bool slot_maps_linear() {
    constexpr int rb = ilog2(R), cb = ilog2(R / 8);
    return gf2::bijective(kc_slot_lin<R>()) && gf2::bijective(mn_slot_lin<R>()) &&
           gf2::agrees(kc_slot_lin<R>(), [](uint32_t x) {
             return (uint32_t)kc_slot((int)(x >> 2), (int)(x & 3));
           }) &&
           gf2::agrees(mn_slot_lin<R>(), [](uint32_t x) {
             return (uint32_t)mn_slot<R>((int)(x >> cb), (int)(x & ((1u << cb) - 1u)));
           }) && rb >= 1;
  }

  // ---- cooperative copies ---------------------------------------------------
  // "My Triton From Scratch, Part 12: CUDA Tile Layouts", section
  // "Cooperative tile layouts": thread t handles linear items t + i*THREADS,
  // ceil(items / THREADS) iterations, the tail lanes of the last one idle.
  // k-contiguous storage: items are 16-byte chunks of the (R, G) grid in
  // order (1, 0) -- g fastest, so 8 neighbouring lanes read one 128-byte
  // run of a row.
  template <int R>
  struct KContig {
    static constexpr int ITEMS = R * G;
    static constexpr int ITERS = (ITEMS + THREADS - 1) / THREADS;
    TRT_HD static bool active(int t, int i) { return t + i * THREADS < ITEMS; }
    TRT_HD static int row(int t, int i) { return (t + i * THREADS) / G; }
    TRT_HD static int g(int t, int i) { return (t + i * THREADS) % G; }
  };
  // Row-contiguous storage (A^T, or row-major B): items are 8x8 blocks of
  // the (R/8, G) grid in order (0, 1) -- the row block fastest, so
  // neighbouring lanes read neighbouring 16-byte runs of one k row.
  template <int R>
  struct MNContig {
    static constexpr int ITEMS = (R / 8) * G;
    static constexpr int ITERS = (ITEMS + THREADS - 1) / THREADS;
    TRT_HD static bool active(int t, int i) { return t + i * THREADS < ITEMS; }
    TRT_HD static int rb(int t, int i) { return (t + i * THREADS) % (R / 8); }
    TRT_HD static int g(int t, int i) { return (t + i * THREADS) / (R / 8); }
  };
};

}  // namespace trt
