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

// Bytes of one element of a dtype: 2 for the 16-bit types, 4 for binary32.
inline int64_t elem_bytes(int32_t dtype) { return dtype == TRT_F32 ? 4 : 2; }

// Bytes spanned by a rows x cols matrix with leading dimension ld (elements
// of `esize` bytes), or false on overflow.
inline bool span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t& bytes,
                       int64_t esize = 2) {
  if (rows <= 0 || cols <= 0) { bytes = 0; return true; }
  const __int128 last = (__int128)(rows - 1) * ld + cols;  // elements
  const __int128 b = last * esize;
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
  if (in_dtype != TRT_F16 && in_dtype != TRT_BF16 && in_dtype != TRT_F32) {
    msg = "in_dtype must be TRT_F16, TRT_BF16 or TRT_F32";
    return TRT_ERR_DTYPE;
  }
  if (out_dtype != TRT_F16 && out_dtype != TRT_BF16 && out_dtype != TRT_F32) {
    msg = "out_dtype must be TRT_F16, TRT_BF16 or TRT_F32";
    return TRT_ERR_DTYPE;
  }
  const bool has_bias = epi && epi->bias;
  const bool has_res = epi && epi->residual;
  const bool has_scale = epi && epi->row_scale;
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
  // every pointer aligned to its element: the input element for A and B,
  // the output element for C and the epilogue operands
  const int64_t isz = elem_bytes(in_dtype), osz = elem_bytes(out_dtype);
  const void* in_ptrs[2] = {A, B};
  const void* out_ptrs[4] = {C, has_bias ? epi->bias : nullptr, has_res ? epi->residual : nullptr,
                             has_scale ? epi->row_scale : nullptr};
  for (const void* q : in_ptrs)
    if (reinterpret_cast<uintptr_t>(q) & (uintptr_t)(isz - 1)) {
      msg = "A and B must be aligned to the input element";
      return TRT_ERR_ALIGN;
    }
  for (const void* q : out_ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & (uintptr_t)(osz - 1))) {
      msg = "C, bias, residual and row_scale must be aligned to the output element";
      return TRT_ERR_ALIGN;
    }
  int64_t sa, sb, sc, sr = 0;
  const bool ok = span_bytes(opA ? K : M, opA ? M : K, lda, sa, isz) &&
                  span_bytes(opB ? N : K, opB ? K : N, ldb, sb, isz) &&
                  span_bytes(M, N, ldc, sc, osz) &&
                  (!has_res || span_bytes(M, N, epi->ldr, sr, osz));
  if (!ok) {
    msg = "operand extent overflows";
    return TRT_ERR_SIZE;
  }
  auto ext = [](const void* q, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Extent{lo, q ? lo + (uintptr_t)bytes : lo};
  };
  const Extent ec = ext(C, sc);
  const Extent ins[5] = {ext(A, sa), ext(B, sb), ext(has_bias ? epi->bias : nullptr, osz * N),
                         ext(has_res ? epi->residual : nullptr, sr),
                         ext(has_scale ? epi->row_scale : nullptr, osz * M)};
  static const char* names[5] = {"A", "B", "bias", "residual", "row_scale"};
  for (int i = 0; i < 5; ++i)
    if (overlaps(ec, ins[i])) {
      msg = std::string("C overlaps ") + names[i] + " (an in-place output is not provably safe)";
      return TRT_ERR_OVERLAP;
    }
  msg.clear();
  return TRT_OK;
}

// The caller's workspace of a call that validate_gemm accepted: at least
// `need` bytes when the call uses one, 16-byte aligned, and disjoint from A,
// B, C and the epilogue operands (the kernels write it while they read the
// inputs, and C is written from it).  A call that needs none accepts any
// workspace, NULL included.
inline trt_status validate_workspace(int64_t M, int64_t N, int64_t K, const void* A,
                                     int64_t lda, int32_t opA, const void* B, int64_t ldb,
                                     int32_t opB, const void* C, int64_t ldc, int32_t in_dtype,
                                     int32_t out_dtype, const trt_epilogue* epi,
                                     const void* ws, int64_t ws_bytes, int64_t need,
                                     std::string& msg) {
  if (need == 0) {
    msg.clear();
    return TRT_OK;
  }
  if (ws_bytes < 0) {
    msg = "workspace_bytes must be >= 0";
    return TRT_ERR_SIZE;
  }
  if (!ws) {
    msg = "this call needs a workspace of " + std::to_string(need) + " bytes";
    return TRT_ERR_NULL;
  }
  if (ws_bytes < need) {
    msg = "the workspace must hold at least " + std::to_string(need) + " bytes";
    return TRT_ERR_SIZE;
  }
  if (reinterpret_cast<uintptr_t>(ws) & 15u) {
    msg = "the workspace must be 16-byte aligned";
    return TRT_ERR_ALIGN;
  }
  const int64_t isz = elem_bytes(in_dtype), osz = elem_bytes(out_dtype);
  const bool has_bias = epi && epi->bias;
  const bool has_res = epi && epi->residual;
  const bool has_scale = epi && epi->row_scale;
  int64_t sa = 0, sb = 0, sc = 0, sr = 0;
  span_bytes(opA ? K : M, opA ? M : K, lda, sa, isz);
  span_bytes(opB ? N : K, opB ? K : N, ldb, sb, isz);
  span_bytes(M, N, ldc, sc, osz);
  if (has_res) span_bytes(M, N, epi->ldr, sr, osz);
  auto ext = [](const void* q, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Extent{lo, q ? lo + (uintptr_t)bytes : lo};
  };
  const Extent ew = ext(ws, need);
  const Extent others[6] = {ext(A, sa), ext(B, sb), ext(C, sc),
                            ext(has_bias ? epi->bias : nullptr, osz * N),
                            ext(has_res ? epi->residual : nullptr, sr),
                            ext(has_scale ? epi->row_scale : nullptr, osz * M)};
  static const char* names[6] = {"A", "B", "C", "bias", "residual", "row_scale"};
  for (int i = 0; i < 6; ++i)
    if (overlaps(ew, others[i])) {
      msg = std::string("the workspace overlaps ") + names[i];
      return TRT_ERR_OVERLAP;
    }
  msg.clear();
  return TRT_OK;
}

}  // namespace trt
