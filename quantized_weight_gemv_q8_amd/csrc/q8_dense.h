// q8_dense.h -- the dense GEMV's row map and epilogue, shared by the
// persistent kernels (q8_gemv.hip) and the one-group-per-wave kernels
// (q8_once*.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_internal.h"

namespace q8 {

// Rows [0, Ma) come from matrix A, rows [Ma, Mtot) from matrix B (the pair).
// Scalar fields and explicit selects: a struct-member select here was
// lowered to a private-memory array.
struct DenseMap {
  const int8_t* qa;
  const uint16_t* da;
  const int8_t* qb;
  const uint16_t* db;
  int64_t ldqa, ldda, ldqb, lddb;
  int64_t Ma, Mtot;
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    const bool second = i >= Ma;
    const int64_t k = second ? i - Ma : i;
    const int64_t ldq = second ? ldqb : ldqa;
    const int64_t ldd = second ? lddb : ldda;
    q = (second ? qb : qa) + k * ldq;
    d = (second ? db : da) + k * ldd;
    return i < Mtot;
  }
};

struct DenseEpi {
  char* ya;
  char* yb;
  int64_t Ma, Mtot;
  bool f16;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (row >= Mtot) continue;
      char* y;
      int64_t col, ld;
      if (row < Ma) { y = ya; col = row; ld = Ma; }
      else { y = yb; col = row - Ma; ld = Mtot - Ma; }
      if (f16) reinterpret_cast<_Float16*>(y)[n * ld + col] = (_Float16)v[i];
      else reinterpret_cast<float*>(y)[n * ld + col] = v[i];
    }
  }
};

// One-group-per-wave launch of a dense pass of nt = 1..8 tokens (weight
// format fmt, lpr lanes per row): hipErrorNotSupported when it does not
// apply (the chunks per lane are not an instantiated count, or, for more
// than 2 tokens, the row groups do not fit in the resident waves); the
// caller then takes the persistent launch.
hipError_t launch_gemv_once(int nt, const DevInfo& dev, const DenseMap& map, const DenseEpi& epi,
                            int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                            hipStream_t s);

}  // namespace q8
