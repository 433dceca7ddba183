/*
 * oracle/gemm_ref.c -- the plain fp64 CPU oracle of the blocked GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no code,
 * header, table or constant with the HIP library and includes nothing from it.
 *
 * What it computes is the plain definition of the operation the pages build:
 *
 *   C(m,n) = epilogue( sum_{k=0}^{K-1} A(m,k) * B(k,n) )
 *
 * "Named layouts" (NineToothed), the GEMM arrangement at the top of the page:
 * an fp32 zero accumulator, acc = acc + dot(lhs[k], rhs[k]) over the K blocks
 * in ascending order, then one cast to the output dtype.  The same page,
 * section "Contract", admits same-output-domain bias / ReLU / residual
 * postprocessing and names the two broadcast operands of a GEMM output: a
 * column bias (axes "n", one value per column) and a row scale (axes "m",
 * one value per row).  The order used here is
 *   relu(acc * scale(m) + bias(n)) + residual(m,n),
 * each term only when present.  Epilogue operands are stored in the output
 * dtype: binary16, bfloat16 or binary32.
 *
 * The oracle takes the sum in fp64 instead of fp32: every product of two
 * 16-bit floats is exact in fp64 (of two binary32 values, within one fp64
 * rounding), and the k order is ascending for every
 * cell, so the result does not depend on thread count or loop nesting.
 * Build with -O2 -ffp-contract=off and without fast-math so that no fused
 * multiply-add or reassociation changes a single rounding.
 *
 * Element addressing follows the explicit-transpose rule ("Named layouts",
 * section "Contract": a transpose is never implied by matching sizes):
 *   opA = 0 : A(m,k) = A[m*lda + k]      opA = 1 : A(m,k) = A[k*lda + m]
 *   opB = 0 : B(k,n) = B[k*ldb + n]      opB = 1 : B(k,n) = B[n*ldb + k]
 *   residual: R(m,n) = R[m*ldr + n]      bias:     bias(n) = bias[n]
 *   row scale: scale(m) = scale[m]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F16 1
#define ORC_BF16 2
#define ORC_F32 3

/* ---- 16-bit formats, decoded from their definitions -------------------- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zeros and subnormals (fraction * 2^-24); field 31
 * holds infinities (fraction 0) and NaNs. */
double orc_decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0)
    v = ldexp((double)frac, -24);
  else if (expo == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(frac + 1024), expo - 25); /* (1 + f/2^10) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Exponent field 0 holds zeros and subnormals (fraction * 2^-133); field 255
 * holds infinities and NaNs. */
double orc_decode_bf16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 7) & 0xff;
  int frac = h & 0x7f;
  double v;
  if (expo == 0)
    v = ldexp((double)frac, -133);
  else if (expo == 255)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(frac + 128), expo - 134); /* (1 + f/2^7) * 2^(e-127) */
  return sign ? -v : v;
}

/* IEEE binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits.
 * Exponent field 0 holds zeros and subnormals (fraction * 2^-149); field 255
 * holds infinities and NaNs. */
double orc_decode_f32(uint32_t w) {
  int sign = (int)((w >> 31) & 1u);
  int expo = (int)((w >> 23) & 0xffu);
  int32_t frac = (int32_t)(w & 0x7fffffu);
  double v;
  if (expo == 0)
    v = ldexp((double)frac, -149);
  else if (expo == 255)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(frac + (1 << 23)), expo - 150); /* (1 + f/2^23) * 2^(e-127) */
  return sign ? -v : v;
}

static double decode(uint16_t h, int dtype) {
  return dtype == ORC_BF16 ? orc_decode_bf16(h) : orc_decode_f16(h);
}

/* Element i of a buffer of the given dtype (16-bit patterns or binary32 words). */
static double decode_at(const void* p, int64_t i, int dtype) {
  if (dtype == ORC_F32) return orc_decode_f32(((const uint32_t*)p)[i]);
  return decode(((const uint16_t*)p)[i], dtype);
}

/* Round an fp64 value to a binary float format, to nearest with ties to
 * even.  frac_bits: 10 (binary16), 7 (bfloat16) or 23 (binary32); emin:
 * -14, -126, -126; emax: 15, 127, 127; exp_bits: 5, 8, 8.  The significand
 * is scaled by a power of two (exact) and rounded with nearbyint() under the
 * default round-to-nearest-even mode.  Returns the bit pattern. */
static uint32_t round_bits(double x, int frac_bits, int emin, int emax, int exp_bits) {
  uint32_t sign = signbit(x) ? (1u << (frac_bits + exp_bits)) : 0u;
  uint32_t inf = ((1u << exp_bits) - 1u) << frac_bits;
  if (isnan(x)) return inf | (1u << (frac_bits - 1)); /* quiet NaN */
  double ax = fabs(x);
  if (isinf(ax)) return sign | inf;
  if (ax == 0.0) return sign;
  int e2;
  (void)frexp(ax, &e2); /* ax = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;       /* ax in [2^E, 2^(E+1)) */
  if (E < emin) {
    /* subnormal range: integer multiples of 2^(emin - frac_bits) */
    double q = nearbyint(ldexp(ax, frac_bits - emin));
    /* q == 2^frac_bits rounds up into the smallest normal, which has the
     * same bit pattern as the fraction overflowing into the exponent. */
    return sign | (uint32_t)q;
  }
  double q = nearbyint(ldexp(ax, frac_bits - E)); /* in [2^fb, 2^(fb+1)] */
  if (q == ldexp(1.0, frac_bits + 1)) {
    q = ldexp(1.0, frac_bits);
    E += 1;
  }
  if (E > emax) return sign | inf;
  uint32_t expo_field = (uint32_t)(E + ((1 << (exp_bits - 1)) - 1));
  uint32_t frac_field = (uint32_t)((int64_t)q - ((int64_t)1 << frac_bits));
  return sign | (expo_field << frac_bits) | frac_field;
}

uint16_t orc_round_f16(double x) { return (uint16_t)round_bits(x, 10, -14, 15, 5); }
uint16_t orc_round_bf16(double x) { return (uint16_t)round_bits(x, 7, -126, 127, 8); }
uint32_t orc_round_f32(double x) { return round_bits(x, 23, -126, 127, 8); }

/* Round n values to `dtype`: 16-bit patterns, or binary32 words for ORC_F32. */
void orc_round_array(const double* x, void* out, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == ORC_F32)
      ((uint32_t*)out)[i] = orc_round_f32(x[i]);
    else
      ((uint16_t*)out)[i] = dtype == ORC_BF16 ? orc_round_bf16(x[i]) : orc_round_f16(x[i]);
  }
}

void orc_decode_array(const void* h, double* out, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = decode_at(h, i, dtype);
}

/* ---- the GEMM and its epilogue ------------------------------------------ */

/* Operand elements: binary16 / bfloat16 patterns, or binary32 words when
 * in_dt is ORC_F32. */
static double elem_a(const void* A, int64_t lda, int opA, int64_t m,
                     int64_t k, int dt) {
  return decode_at(A, opA ? k * lda + m : m * lda + k, dt);
}

static double elem_b(const void* B, int64_t ldb, int opB, int64_t k,
                     int64_t n, int dt) {
  return decode_at(B, opB ? n * ldb + k : k * ldb + n, dt);
}

/* Epilogue of one cell, in fp64: y = acc; y *= scale(m); y += bias(n);
 * y = max(y, 0); y += R(m,n).  Each step only when its operand or flag is
 * present; scale, bias and R hold elements of the output dtype out_dt. */
static double epilogue(double acc, int64_t m, int64_t n, const void* scale,
                       const void* bias, int relu, const void* R, int64_t ldr,
                       int out_dt) {
  double y = acc;
  if (scale) y *= decode_at(scale, m, out_dt);
  if (bias) y += decode_at(bias, n, out_dt);
  if (relu) y = y > 0.0 ? y : 0.0;
  if (R) y += decode_at(R, m * ldr + n, out_dt);
  return y;
}

/*
 * Reference values of the block [m_lo, m_hi) x [n_lo, n_hi) of C, written to
 * out[(m - m_lo) * (n_hi - n_lo) + (n - n_lo)] unrounded (fp64).
 *
 * Each row is an independent job (OpenMP over rows when nthreads > 1).  For a
 * row, the accumulators of all its cells start at zero and receive the terms
 * k = 0, 1, ..., K-1 in that order; walking k in the outer loop and n in the
 * inner loop does not change the order of any single cell's sum.
 * Returns 0, or -1 on an argument error.
 */
int orc_gemm_block(int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, int opA, const void* B, int64_t ldb,
                   int opB, int in_dt, const void* scale, const void* bias,
                   int relu, const void* R, int64_t ldr, int out_dt, int64_t m_lo,
                   int64_t m_hi, int64_t n_lo, int64_t n_hi, double* out,
                   int nthreads) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  if (m_lo < 0 || m_hi > M || m_lo >= m_hi) return -1;
  if (n_lo < 0 || n_hi > N || n_lo >= n_hi) return -1;
  int64_t W = n_hi - n_lo;
  /* Decode B's needed columns once per call: Bd[k][n - n_lo]. */
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * W));
  if (!Bd) return -1;
  for (int64_t k = 0; k < K; ++k)
    for (int64_t n = n_lo; n < n_hi; ++n)
      Bd[k * W + (n - n_lo)] = elem_b(B, ldb, opB, k, n, in_dt);

#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t m = m_lo; m < m_hi; ++m) {
    double* acc = out + (m - m_lo) * W;
    for (int64_t j = 0; j < W; ++j) acc[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = elem_a(A, lda, opA, m, k, in_dt);
      const double* brow = Bd + k * W;
      for (int64_t j = 0; j < W; ++j) acc[j] += a * brow[j];
    }
    for (int64_t j = 0; j < W; ++j)
      acc[j] = epilogue(acc[j], m, n_lo + j, scale, bias, relu, R, ldr, out_dt);
  }
  free(Bd);
  return 0;
}

/* Reference values of scattered cells (ms[i], ns[i]), one by one, with the
 * same per-cell order (k ascending).  Used to sample outputs of shapes too
 * large for a full oracle run. */
int orc_gemm_cells(int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, int opA, const void* B, int64_t ldb,
                   int opB, int in_dt, const void* scale, const void* bias,
                   int relu, const void* R, int64_t ldr, int out_dt,
                   const int64_t* ms, const int64_t* ns, int64_t count,
                   double* out, int nthreads) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
  for (int64_t i = 0; i < count; ++i) {
    int64_t m = ms[i], n = ns[i];
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
      acc += elem_a(A, lda, opA, m, k, in_dt) * elem_b(B, ldb, opB, k, n, in_dt);
    out[i] = epilogue(acc, m, n, scale, bias, relu, R, ldr, out_dt);
  }
  return 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
