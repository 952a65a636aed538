// q8_q4.hip -- dense Q4_0 GEMV (gfx950).
//
// The pages decode Q4_0 weights with the same split-plane matvecs as Q8_0
// (memra wiki, feature list: "NVFP4 / Q4_0 / Q8_0 decode ... split-plane
// repacked matvecs"; memra performance: "wide-load Q4_0 expert dots"). A
// GGUF Q4_0 block holds an fp16 scale and 16 bytes of 4-bit values stored
// with +8: the low nibble of byte j is element j, the high nibble element
// j + 16. The packed layout keeps those 16 bytes as they are in a nibble
// plane (row stride >= K/2 bytes) next to the fp16 scale plane, so one
// 16-byte load is exactly one block: 32 weights and one scale. Half the
// bytes of Q8_0 per weight, twice the arithmetic per byte.
//
// Arithmetic per (row, token) mirrors the Q8_0 engine: each nibble becomes
// the exact fp16 value 1024 + (q + 8) by placing it under an exponent byte
// of 0x64 and 1032 is subtracted (integers below 2048, exact); the 32
// products with the fp16 activations are summed by v_dot2_f32_f16 in K
// order, scaled by fp32(d) with one FMA per block, and the team's partials
// meet in the engine's fixed butterfly. The order does not depend on N, R
// or the other tokens, so results are bitwise N-invariant.
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

// One Q4_0 block (16 bytes) -> 16 fp16 pairs in element order: pairs 0..7
// from the low nibbles (elements 0..15), 8..15 from the high nibbles.
__device__ __forceinline__ void nibbles_to_h2(const uint4 q, h2_t out[16]) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
  const h2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned lo = w[i] & 0x0F0F0F0Fu;
    const unsigned hi = (w[i] >> 4) & 0x0F0F0F0Fu;
    out[2 * i] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - bias;
    out[2 * i + 1] =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - bias;
    out[8 + 2 * i] =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - bias;
    out[8 + 2 * i + 1] =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - bias;
  }
}

// sum_{i<32} q_i * x_i in fp32, sequential over the 16 pairs in K order;
// x0..x3 hold elements 0-7, 8-15, 16-23 and 24-31.
__device__ __forceinline__ float dot32_f16(const h2_t q[16], const uint4 x0, const uint4 x1,
                                           const uint4 x2, const uint4 x3) {
  const uint4 xs[4] = {x0, x1, x2, x3};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = __builtin_amdgcn_fdot2(q[4 * i + 0], __builtin_bit_cast(h2_t, xs[i].x), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 1], __builtin_bit_cast(h2_t, xs[i].y), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 2], __builtin_bit_cast(h2_t, xs[i].z), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 3], __builtin_bit_cast(h2_t, xs[i].w), s, false);
  }
  return s;
}

// fp32 activations: nibble - 8 as fp32 (exact), then an FMA chain in K order.
__device__ __forceinline__ float dot32_f32(const uint4 q, const uint4* x) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
  float s = 0.0f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xv = __builtin_bit_cast(float4, x[half * 4 + i]);
      const float xe[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int nib = (int)((w[i] >> (8 * b + 4 * half)) & 0xFu) - 8;
        s = __builtin_fmaf((float)nib, xe[b], s);
      }
    }
  }
  return s;
}

template <bool XF32>
struct Q4Planes {
  static constexpr int P = XF32 ? 8 : 4;  // 16-byte pieces of x per block
};

struct Q4Map {
  const uint8_t* qs;
  const uint16_t* d;
  int64_t ldq, ldd, M;
  __device__ __forceinline__ bool row(int64_t i, const uint8_t*& q, const uint16_t*& dd) const {
    q = qs + i * ldq;
    dd = d + i * ldd;
    return i < M;
  }
};

struct Q4Epi {
  char* y;
  int64_t M;
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
      if (row >= M) continue;
      if (f16) reinterpret_cast<_Float16*>(y)[n * M + row] = (_Float16)v[i];
      else reinterpret_cast<float*>(y)[n * M + row] = v[i];
    }
  }
};

// The engine's row loop for 16-byte Q4_0 blocks: team lane p takes blocks
// p, p + LPR, ... of its R rows; one block load ahead (the window measured
// best for Q8_0); row pointers refreshed once per group.
template <int NT, int LPR, int R, bool XF32, class Map, class Epi, class Stage>
__device__ __forceinline__ void run_rows_q4(const Map& map, Epi& epi, const uint4* lds, int C,
                                            int64_t n_groups, int64_t g_first, int64_t g_stride,
                                            Stage&& stage) {
  constexpr int RPW = kWave / LPR;
  constexpr int G = RPW * R;
  constexpr int V = NT * R;
  constexpr int VP = Pow2<V>::value;
  using Shape = ReduceShape<LPR, VP, 1>;
  constexpr int P = Q4Planes<XF32>::P;

  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane % LPR;
  const int team = lane / LPR;
  const int CPL = (C + LPR - 1) / LPR;
  const int64_t my_groups = g_first < n_groups ? (n_groups - g_first + g_stride - 1) / g_stride : 0;
  const int64_t total = my_groups * CPL;

  uint4 sq[R];
  uint16_t sd[R];
  int64_t ig = g_first;
  int ij = 0;
  const uint8_t* iq[R];
  const uint16_t* id[R];
  bool iok[R];
  auto refresh = [&]() {
    const bool live = ig < n_groups;
    const int64_t rbase = ig * G + (int64_t)team * R;
#pragma unroll
    for (int r = 0; r < R; ++r) iok[r] = live && map.row(rbase + r, iq[r], id[r]);
  };
  refresh();
  auto issue = [&]() {
    const int c = p + LPR * ij;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (iok[r] && c < C) {
        sq[r] = load_stream16(reinterpret_cast<const int8_t*>(iq[r]) + (int64_t)c * 16);
        sd[r] = id[r][c];
      } else {
        sq[r] = make_uint4(0, 0, 0, 0);
        sd[r] = 0;
      }
    }
    if (++ij == CPL) {
      ij = 0;
      ig += g_stride;
      refresh();
    }
  };

  issue();
  stage();

  float acc[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
  int64_t cg = g_first;
  int cj = 0;
  for (int64_t it = 0; it < total; ++it) {
    const int c = p + LPR * cj;
    if (c < C) {
      float df[R];
#pragma unroll
      for (int r = 0; r < R; ++r) df[r] = half_bits_to_float(sd[r]);
      if constexpr (!XF32) {
        h2_t qh[R][16];
#pragma unroll
        for (int r = 0; r < R; ++r) nibbles_to_h2(sq[r], qh[r]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint4 x0 = lds[(n * P + 0) * C + c];
          const uint4 x1 = lds[(n * P + 1) * C + c];
          const uint4 x2 = lds[(n * P + 2) * C + c];
          const uint4 x3 = lds[(n * P + 3) * C + c];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float sum = dot32_f16(qh[r], x0, x1, x2, x3);
            acc[n * R + r] = __builtin_fmaf(df[r], sum, acc[n * R + r]);
          }
        }
      } else {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          uint4 xv[8];
#pragma unroll
          for (int h = 0; h < 8; ++h) xv[h] = lds[(n * P + h) * C + c];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float sum = dot32_f32(sq[r], xv);
            acc[n * R + r] = __builtin_fmaf(df[r], sum, acc[n * R + r]);
          }
        }
      }
    }
    issue();
    if (++cj == CPL) {
      if (cg < n_groups) {
        int base = 0;
        TeamReduce<VP, 1, LPR / 2>::run(acc, p, base);
        const bool owner = (p & Shape::OWNER_MASK) == 0;
        epi.template emit<NT, R, Shape::CNT>(cg * G + (int64_t)team * R, base, owner, acc);
      }
#pragma unroll
      for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
      cj = 0;
      cg += g_stride;
    }
  }
}

template <int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(kBlock) void gemv_q4_kernel(Q4Map map, Q4Epi epi, const char* x,
                                                         int64_t ldx_bytes, int C) {
  extern __shared__ uint4 lds_x[];
  constexpr int R = Tune<NT, BIG>::R;
  constexpr int G = (kWave / LPR) * R;
  const int64_t n_groups = (map.M + G - 1) / G;
  const int wave = threadIdx.x / kWave;
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
    stage_planes<NT, Q4Planes<XF32>::P>(rows, C, lds_x);
    __syncthreads();
  };
  run_rows_q4<NT, LPR, R, XF32>(map, epi, lds_x, C, n_groups,
                                (int64_t)blockIdx.x * kWavesPerBlock + wave,
                                (int64_t)gridDim.x * kWavesPerBlock, stage);
}

template <int NT, int LPR, bool XF32, bool BIG>
static hipError_t q4_launch_t(const DevInfo& dev, Q4Map map, Q4Epi epi, const char* x,
                              int64_t ldx_bytes, int C, hipStream_t s) {
  constexpr int G = (kWave / LPR) * Tune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * Q4Planes<XF32>::P;
  const int64_t n_groups = (map.M + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  auto fn = gemv_q4_kernel<NT, LPR, XF32, BIG>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
}

template <int LPR, bool XF32>
static hipError_t q4_launch_nt(const DevInfo& dev, int nt, Q4Map map, Q4Epi epi, const char* x,
                               int64_t ldx_bytes, int C, hipStream_t s) {
  switch (nt) {
    case 1:
      if (map.M >= kBigRows) return q4_launch_t<1, LPR, XF32, true>(dev, map, epi, x, ldx_bytes, C, s);
      return q4_launch_t<1, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 2: return q4_launch_t<2, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 3: return q4_launch_t<3, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 4: return q4_launch_t<4, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 5: return q4_launch_t<5, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 6: return q4_launch_t<6, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 7: return q4_launch_t<7, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 8: return q4_launch_t<8, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_q4(const DevInfo& dev, const HMat& W, const void* x, bool x_f32, void* y,
                          bool y_f16, int nt, hipStream_t s) {
  Q4Map map;
  map.qs = reinterpret_cast<const uint8_t*>(W.qs);
  map.d = W.d;
  map.ldq = W.ld_qs;
  map.ldd = W.ld_d;
  map.M = W.M;
  Q4Epi epi;
  epi.y = (char*)y;
  epi.M = W.M;
  epi.f16 = y_f16;
  const int C = (int)(W.K / 32);  // one 16-byte block per chunk
  const int64_t ldx_bytes = W.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int lpr = lanes_per_row(W.K / 2);  // lanes from the number of 16-byte chunks
  if (x_f32) {
    if (lpr == 64) return q4_launch_nt<64, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
    if (lpr == 32) return q4_launch_nt<32, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
    return q4_launch_nt<16, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  }
  if (lpr == 64) return q4_launch_nt<64, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  if (lpr == 32) return q4_launch_nt<32, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  return q4_launch_nt<16, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
}

}  // namespace q8
