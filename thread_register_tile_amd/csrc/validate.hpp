// validate.hpp -- host-side argument checks of the GEMM entry points.
//
// NineToothed "Named layouts", section "Runtime and compilation": logical
// sizes must be positive, input strides positive (non-contiguous inputs are
// allowed), output writes provably non-overlapping, output storage disjoint
// from every input; the checks run before any kernel work, and a case whose
// safety cannot be proven is an error.  Pure C++: no HIP call, no pointer
// dereference, so it can run (and be tested) on a machine without a GPU.
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/trt.h"

namespace trt {

// Largest extent accepted for M, N, K: index arithmetic in the kernels uses
// 32-bit tile coordinates and 64-bit element offsets.
constexpr int64_t kMaxDim = int64_t(1) << 30;

struct Extent {
  uintptr_t lo, hi;  // [lo, hi) in bytes; lo == hi for an absent buffer
};

// Bytes spanned by a rows x cols matrix with leading dimension ld (elements
// of 2 bytes), or false on overflow.
inline bool span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t& bytes) {
  if (rows <= 0 || cols <= 0) { bytes = 0; return true; }
  const __int128 last = (__int128)(rows - 1) * ld + cols;  // elements
  const __int128 b = last * 2;
  if (b > ((__int128)1 << 62)) return false;
  bytes = (int64_t)b;
  return true;
}

inline bool overlaps(Extent a, Extent b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

inline trt_status validate_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                int32_t opA, const void* B, int64_t ldb, int32_t opB,
                                const void* C, int64_t ldc, int32_t in_dtype,
                                int32_t out_dtype, const trt_epilogue* epi,
                                std::string& msg) {
  if (M < 1 || N < 1 || K < 1) {
    msg = "M, N and K must be >= 1";
    return TRT_ERR_SIZE;
  }
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) {
    msg = "M, N and K must be <= 2^30";
    return TRT_ERR_SIZE;
  }
  if (opA != TRT_OP_N && opA != TRT_OP_T) {
    msg = "opA must be TRT_OP_N or TRT_OP_T";
    return TRT_ERR_ARG;
  }
  if (opB != TRT_OP_N && opB != TRT_OP_T) {
    msg = "opB must be TRT_OP_N or TRT_OP_T";
    return TRT_ERR_ARG;
  }
  if (in_dtype != TRT_F16 && in_dtype != TRT_BF16) {
    msg = "in_dtype must be TRT_F16 or TRT_BF16";
    return TRT_ERR_DTYPE;
  }
  if (out_dtype != in_dtype) {
    msg = "out_dtype must equal in_dtype";
    return TRT_ERR_DTYPE;
  }
  const bool has_bias = epi && epi->bias;
  const bool has_res = epi && epi->residual;
  if (lda < 1 || ldb < 1 || (has_res && epi->ldr < 1)) {
    msg = "input leading dimensions must be >= 1";
    return TRT_ERR_STRIDE;
  }
  if (ldc < N) {
    msg = "ldc must be >= N so that output rows do not overlap";
    return TRT_ERR_STRIDE;
  }
  if (!A || !B || !C) {
    msg = "A, B and C must be non-null";
    return TRT_ERR_NULL;
  }
  const void* ptrs[5] = {A, B, C, has_bias ? epi->bias : nullptr,
                         has_res ? epi->residual : nullptr};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 1u)) {
      msg = "pointers must be 2-byte aligned";
      return TRT_ERR_ALIGN;
    }
  int64_t sa, sb, sc, sr = 0;
  const bool ok = span_bytes(opA ? K : M, opA ? M : K, lda, sa) &&
                  span_bytes(opB ? N : K, opB ? K : N, ldb, sb) &&
                  span_bytes(M, N, ldc, sc) &&
                  (!has_res || span_bytes(M, N, epi->ldr, sr));
  if (!ok) {
    msg = "operand extent overflows";
    return TRT_ERR_SIZE;
  }
  auto ext = [](const void* q, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Extent{lo, q ? lo + (uintptr_t)bytes : lo};
  };
  const Extent ec = ext(C, sc);
  const Extent ins[4] = {ext(A, sa), ext(B, sb), ext(has_bias ? epi->bias : nullptr, 2 * N),
                         ext(has_res ? epi->residual : nullptr, sr)};
  static const char* names[4] = {"A", "B", "bias", "residual"};
  for (int i = 0; i < 4; ++i)
    if (overlaps(ec, ins[i])) {
      msg = std::string("C overlaps ") + names[i] + " (an in-place output is not provably safe)";
      return TRT_ERR_OVERLAP;
    }
  msg.clear();
  return TRT_OK;
}

}  // namespace trt
