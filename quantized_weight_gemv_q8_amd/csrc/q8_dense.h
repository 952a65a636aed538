// q8_dense.h -- the row maps and epilogues of the dense GEMV and of the
// gate/up + SiLU pair, shared by the persistent kernels (q8_gemv.hip) and
// the one-group-per-wave kernels (q8_once*.hip).
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
  int nt = kMaxNTWide;  // live tokens: only a kernel whose token count is a runtime value sets it
  // Gated accumulate (the shared expert's last step): with gate set, y is
  // fp32 and read-modify-written, y[n][m] += sigmoid(gate[n]) * v, with
  // sigmoid(z) = 1 / (1 + expf(-z)); gate[n] is the raw gate dot of token n.
  const float* gate = nullptr;
  // Token slice of a launch that runs several passes at once: token n of
  // the slice starting at token n0 is token n0 + n of the call.
  __device__ __forceinline__ void shift(int n0) {
    const int64_t es = f16 && gate == nullptr ? 2 : 4;
    ya += (int64_t)n0 * Ma * es;
    if (yb != nullptr) yb += (int64_t)n0 * (Mtot - Ma) * es;
    if (gate != nullptr) gate += n0;
  }
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (row >= Mtot || n >= nt) continue;
      char* y;
      int64_t col, ld;
      if (row < Ma) { y = ya; col = row; ld = Ma; }
      else { y = yb; col = row - Ma; ld = Mtot - Ma; }
      if (gate) {
        float* o = reinterpret_cast<float*>(y) + n * ld + col;
        const float g = 1.0f / (1.0f + expf(-gate[n]));
        *o = __builtin_fmaf(g, v[i], *o);
      } else if (f16) {
        reinterpret_cast<_Float16*>(y)[n * ld + col] = (_Float16)v[i];
      } else {
        reinterpret_cast<float*>(y)[n * ld + col] = v[i];
      }
    }
  }
};

// The gate and up rows of output rho are virtual rows 2*rho and 2*rho + 1,
// so a team (an even number of rows) holds both sums of an output in one
// lane after the reduction and the MLP activation h = silu(g) * u is
// applied before anything is stored. Per-row arithmetic is the engine's, so
// g and u are bitwise those of q8_gemv_pair.
struct GluMap {
  const int8_t* qg;
  const uint16_t* dg;
  const int8_t* qu;
  const uint16_t* du;
  int64_t ldqg, lddg, ldqu, lddu;
  int64_t M2;  // 2 * M virtual rows, 2 * M + 2 with an extra row
  // Optional extra row (the shared expert's gate row, one row of the same
  // K): virtual rows 2M and 2M + 1 both read it, so its dot with x lands in
  // the lane that would hold an output's gate and up sums.
  const int8_t* qx = nullptr;
  const uint16_t* dx = nullptr;
  int64_t M = 0;
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    const int64_t rho = i >> 1;
    const bool up = (i & 1) != 0;
    const int64_t ldq = up ? ldqu : ldqg;
    const int64_t ldd = up ? lddu : lddg;
    q = (up ? qu : qg) + rho * ldq;
    d = (up ? du : dg) + rho * ldd;
    if (qx != nullptr && rho == M) {
      q = qx;
      d = dx;
    }
    return i < M2;
  }
};

struct GluEpi {
  char* h;
  int64_t M;
  bool f16;
  int nt = kMaxNTWide;  // live tokens, as for DenseEpi
  float* xdot = nullptr;  // with an extra row: its dot with token n goes to xdot[n]
  __device__ __forceinline__ void shift(int n0) {  // as DenseEpi::shift
    h += (int64_t)n0 * M * (f16 ? 2 : 4);
    if (xdot != nullptr) xdot += n0;
  }
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    static_assert(R % 2 == 0 && CNT == 2, "gate/up pairs");
    if (!owner || base >= NT * R) return;
    const int n = base / R, r = base - (base / R) * R;
    const int64_t row = rbase + r;  // the gate row of the pair (even)
    if (n >= nt) return;
    if (row >= 2 * M) {
      if (xdot != nullptr && row == 2 * M) xdot[n] = v[0];
      return;
    }
    const float g = v[0], u = v[1];
    const float val = g / (1.0f + expf(-g)) * u;
    const int64_t o = (int64_t)n * M + (row >> 1);
    if (f16) reinterpret_cast<_Float16*>(h)[o] = (_Float16)val;
    else reinterpret_cast<float*>(h)[o] = val;
  }
};

// One-group-per-wave launch of a dense pass of nt = 1..8 tokens (weight
// format fmt, lpr lanes per row): hipErrorNotSupported when it does not
// apply (the chunks per lane are not an instantiated count, or, for more
// than 2 tokens, the row groups do not fit in the resident waves); the
// caller then takes the persistent launch.
// With slices > 1 the launch runs that many passes of nt tokens at once
// (blockIdx.y is the pass; pass k reads x + k * nt * ldx_bytes and writes
// tokens k * nt ..): the weights are streamed from HBM by the first pass
// and mostly found in the L2 by the others.
hipError_t launch_gemv_once(int nt, const DevInfo& dev, const DenseMap& map, const DenseEpi& epi,
                            int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                            hipStream_t s, int slices = 1);

// The same for the gate/up + SiLU pair (2M virtual rows), nt = 1..8 (from
// 3 tokens only when every group fits in the resident waves).
hipError_t launch_glu_once(int nt, const DevInfo& dev, const GluMap& map, const GluEpi& epi,
                           int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                           hipStream_t s, int slices = 1);

}  // namespace q8
