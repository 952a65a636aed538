// q8_engine.hpp -- device core shared by every Q8_0 GEMV kernel (gfx950).
//
// The decode matvec is bound by HBM: each weight byte is used once per
// token, so the kernel's job is to stream the quant and scale planes at the
// memory system's rate and keep everything else off the critical path
// (memra wiki: plain decode "sits at the DRAM wall"; memra performance,
// "Dense IQ4_XS qmatvec arm 1": wide aligned loads relieve the load queue).
//
// Work decomposition (wave64):
//  * A row is cut into 16-byte chunks (16 quants = half a Q8_0 block).
//    A team of LPR lanes (64, 32 or 16, chosen from K only) owns a row;
//    lane p of the team handles chunks c = p, p+LPR, p+2*LPR, ... so each
//    load instruction of a 64-lane team reads 1 KiB of contiguous quants
//    (global_load_dwordx4, coalesced), plus the chunk's fp16 scale.
//  * A team processes R rows at once ("group"); the quants of a chunk are
//    converted once and reused for all NT tokens and the x value of a chunk
//    is read once from LDS and reused for all R rows.
//  * x (all NT tokens) is staged once per workgroup into LDS, split into
//    16-byte planes so that consecutive lanes read consecutive 16-byte LDS
//    words.
//
// Arithmetic (per row, token): each int8 becomes an exact fp16 value
// (q in [-128, 127] is representable), the 16 products with the fp16
// activations are summed by v_dot2_f32_f16 in fp32 (every product of an
// 8-bit integer and an fp16 is exact in fp32), the chunk sum is scaled by
// the block's fp32(d) with one FMA into the lane's accumulator, and the
// team's partials are combined by a fixed butterfly. Nothing in this
// sequence depends on N, on R, or on the other tokens, so every token's
// result is bitwise identical whatever the batch (memra wiki gate
// paragraph: K=1..8 speculative verify must equal plain decode; "FP
// summation order is part of the contract").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 512;  // threads per workgroup for every row kernel
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxNT = 8;    // tokens per pass

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// 16 int8 quants (K order, little-endian bytes of a uint4) -> 8 fp16 pairs.
// Each byte b is flipped to excess-128 (u = b ^ 0x80 = q + 128), placed as the
// low mantissa byte of the fp16 value 1024 + u (exponent field 0x64 gives
// 1024 with a unit ulp), and 1152 is subtracted: (1024 + q + 128) - 1152 = q,
// exact because every intermediate is an integer below 2048.
__device__ __forceinline__ void quants_to_h2(const uint4 q, h2_t out[8]) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
  const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned u = w[i] ^ 0x80808080u;
    const unsigned lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const unsigned hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    out[2 * i] = __builtin_bit_cast(h2_t, lo) - bias;
    out[2 * i + 1] = __builtin_bit_cast(h2_t, hi) - bias;
  }
}

// sum_{i<16} q_i * x_i in fp32, sequential over the 8 pairs in K order.
__device__ __forceinline__ float dot16_f16(const h2_t q[8], const uint4 xlo, const uint4 xhi) {
  float s = 0.0f;
  s = __builtin_amdgcn_fdot2(q[0], __builtin_bit_cast(h2_t, xlo.x), s, false);
  s = __builtin_amdgcn_fdot2(q[1], __builtin_bit_cast(h2_t, xlo.y), s, false);
  s = __builtin_amdgcn_fdot2(q[2], __builtin_bit_cast(h2_t, xlo.z), s, false);
  s = __builtin_amdgcn_fdot2(q[3], __builtin_bit_cast(h2_t, xlo.w), s, false);
  s = __builtin_amdgcn_fdot2(q[4], __builtin_bit_cast(h2_t, xhi.x), s, false);
  s = __builtin_amdgcn_fdot2(q[5], __builtin_bit_cast(h2_t, xhi.y), s, false);
  s = __builtin_amdgcn_fdot2(q[6], __builtin_bit_cast(h2_t, xhi.z), s, false);
  s = __builtin_amdgcn_fdot2(q[7], __builtin_bit_cast(h2_t, xhi.w), s, false);
  return s;
}

// 16 int8 quants -> fp32 (sign-extending byte converts, exact).
__device__ __forceinline__ void quants_to_f32(const uint4 q, float out[16]) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) out[4 * i + b] = (float)(int8_t)(w[i] >> (8 * b));
  }
}

// sum_{i<16} q_i * x_i with fp32 activations: sequential fp32 FMAs in K order.
__device__ __forceinline__ float dot16_f32(const float q[16], const float4 x0, const float4 x1,
                                           const float4 x2, const float4 x3) {
  float s = 0.0f;
  s = __builtin_fmaf(q[0], x0.x, s);
  s = __builtin_fmaf(q[1], x0.y, s);
  s = __builtin_fmaf(q[2], x0.z, s);
  s = __builtin_fmaf(q[3], x0.w, s);
  s = __builtin_fmaf(q[4], x1.x, s);
  s = __builtin_fmaf(q[5], x1.y, s);
  s = __builtin_fmaf(q[6], x1.z, s);
  s = __builtin_fmaf(q[7], x1.w, s);
  s = __builtin_fmaf(q[8], x2.x, s);
  s = __builtin_fmaf(q[9], x2.y, s);
  s = __builtin_fmaf(q[10], x2.z, s);
  s = __builtin_fmaf(q[11], x2.w, s);
  s = __builtin_fmaf(q[12], x3.x, s);
  s = __builtin_fmaf(q[13], x3.y, s);
  s = __builtin_fmaf(q[14], x3.z, s);
  s = __builtin_fmaf(q[15], x3.w, s);
  return s;
}

// ---------------------------------------------------------------- x staging
// LDS image of x for one pass: token n, plane h (16-byte piece h of a chunk:
// 2 planes for fp16, 4 for fp32), chunk c at uint4 index (n*P + h)*C + c.
template <bool XF32>
struct XPlanes {
  static constexpr int P = XF32 ? 4 : 2;
};

// rows[n] points at token n's K activations (16-byte aligned).
template <int NT, bool XF32>
__device__ __forceinline__ void stage_x(const char* const rows[NT], int C, uint4* lds) {
  constexpr int P = XPlanes<XF32>::P;
  const int per_tok = C * P;
  for (int n = 0; n < NT; ++n) {
    const uint4* src = reinterpret_cast<const uint4*>(rows[n]);
    for (int i = threadIdx.x; i < per_tok; i += blockDim.x) {
      const int c = i / P, h = i - c * P;
      lds[(n * P + h) * C + c] = src[i];
    }
  }
}

// ---------------------------------------------------------------- team reduction
// Butterfly over the LPR lanes of a team, xor distances LPR/2, LPR/4, ..., 1.
// While a lane carries more than MINC values, each level halves them
// (the lane keeps the half selected by its distance bit and receives the
// partner's copy of that half), so R*NT sums cost about R*NT shuffles
// instead of log2(LPR) each. Every value is summed over the same pairing
// tree (partners differing in bit LPR/2, then LPR/4, ...), whatever the
// number of values carried, so the result of each (row, token) does not
// depend on R or NT. fp32 addition is commutative, so the side a value
// arrives from does not matter.
template <int CNT, int MINC, int DELTA>
struct TeamReduce {
  static __device__ __forceinline__ void run(float* v, int p, int& base) {
    if constexpr (DELTA == 0) {
      return;
    } else if constexpr (CNT > MINC) {
      constexpr int H = CNT / 2;
      const bool hi = (p & DELTA) != 0;
      float nv[H];
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = hi ? v[i] : v[i + H];
        const float keep = hi ? v[i + H] : v[i];
        nv[i] = keep + __shfl_xor(send, DELTA, kWave);
      }
#pragma unroll
      for (int i = 0; i < H; ++i) v[i] = nv[i];
      if (hi) base += H;
      TeamReduce<H, MINC, DELTA / 2>::run(v, p, base);
    } else {
#pragma unroll
      for (int i = 0; i < CNT; ++i) v[i] = v[i] + __shfl_xor(v[i], DELTA, kWave);
      TeamReduce<CNT, MINC, DELTA / 2>::run(v, p, base);
    }
  }
};

template <int V>
struct Pow2 {
  static constexpr int value = V <= 1 ? 1 : 2 * Pow2<(V + 1) / 2>::value;
};

// Number of values left per lane and number of halving levels.
template <int LPR, int VP, int MINC>
struct ReduceShape {
  static constexpr int levels() {
    int l = 0, c = VP, d = LPR / 2;
    while (d > 0 && c > MINC) { c /= 2; d /= 2; ++l; }
    return l;
  }
  static constexpr int L = levels();
  static constexpr int CNT = VP >> L;
  // lanes whose low bits (the all-reduce levels) are zero own their values
  static constexpr int OWNER_MASK = (LPR >> L) - 1;
};

// ---------------------------------------------------------------- row sources
struct MatDesc {
  const int8_t* qs;
  const uint16_t* d;
  int64_t ld_qs;  // bytes
  int64_t ld_d;   // fp16 elements
};

// ---------------------------------------------------------------- engine
// Processes groups of rows [row0, row0 + G) for g = g_first, g_first +
// g_stride, ... < n_groups. map.row(i, q, d) gives row i's planes (false if
// the row does not exist). epi.emit(row_base, base, cnt, owner, v) receives
// the reduced sums: values v[0..cnt) are (token n, row r) pairs with flat
// index base+i = n*R + r, rows row_base + r.
template <int NT, int LPR, int R, int MINC, bool XF32, class Map, class Epi>
__device__ __forceinline__ void run_rows(const Map& map, Epi& epi, const uint4* lds, int C,
                                         int64_t n_groups, int64_t g_first, int64_t g_stride,
                                         int64_t row_origin) {
  constexpr int RPW = kWave / LPR;  // teams per wave
  constexpr int G = RPW * R;        // rows per wave per group
  constexpr int V = NT * R;
  constexpr int VP = Pow2<V>::value;
  using Shape = ReduceShape<LPR, VP, MINC>;
  constexpr int P = XPlanes<XF32>::P;

  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane % LPR;
  const int team = lane / LPR;
  const int CPL = (C + LPR - 1) / LPR;

  for (int64_t g = g_first; g < n_groups; g += g_stride) {
    const int64_t rbase = row_origin + g * G + (int64_t)team * R;
    const int8_t* qp[R];
    const uint16_t* dp[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ok[r] = map.row(rbase + r, qp[r], dp[r]);

    float acc[VP];
#pragma unroll
    for (int i = 0; i < VP; ++i) acc[i] = 0.0f;

    uint4 qn[R];
    uint16_t dn[R];
    {
      const int c = p;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (ok[r] && c < C) {
          qn[r] = *reinterpret_cast<const uint4*>(qp[r] + (int64_t)c * 16);
          dn[r] = dp[r][c >> 1];
        } else {
          qn[r] = make_uint4(0, 0, 0, 0);
          dn[r] = 0;
        }
      }
    }
    for (int j = 0; j < CPL; ++j) {
      uint4 qc[R];
      uint16_t dc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) { qc[r] = qn[r]; dc[r] = dn[r]; }
      const int cn = p + LPR * (j + 1);
      if (j + 1 < CPL) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (ok[r] && cn < C) {
            qn[r] = *reinterpret_cast<const uint4*>(qp[r] + (int64_t)cn * 16);
            dn[r] = dp[r][cn >> 1];
          } else {
            qn[r] = make_uint4(0, 0, 0, 0);
            dn[r] = 0;
          }
        }
      }
      const int c = p + LPR * j;
      if (c < C) {
        float df[R];
#pragma unroll
        for (int r = 0; r < R; ++r) df[r] = half_bits_to_float(dc[r]);
        if constexpr (!XF32) {
          h2_t qh[R][8];
#pragma unroll
          for (int r = 0; r < R; ++r) quants_to_h2(qc[r], qh[r]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const uint4 xlo = lds[(n * P + 0) * C + c];
            const uint4 xhi = lds[(n * P + 1) * C + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const float s = dot16_f16(qh[r], xlo, xhi);
              acc[n * R + r] = __builtin_fmaf(df[r], s, acc[n * R + r]);
            }
          }
        } else {
          float qf[R][16];
#pragma unroll
          for (int r = 0; r < R; ++r) quants_to_f32(qc[r], qf[r]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const uint4 a = lds[(n * P + 0) * C + c];
            const uint4 b = lds[(n * P + 1) * C + c];
            const uint4 e = lds[(n * P + 2) * C + c];
            const uint4 f = lds[(n * P + 3) * C + c];
            const float4 x0 = __builtin_bit_cast(float4, a);
            const float4 x1 = __builtin_bit_cast(float4, b);
            const float4 x2 = __builtin_bit_cast(float4, e);
            const float4 x3 = __builtin_bit_cast(float4, f);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const float s = dot16_f32(qf[r], x0, x1, x2, x3);
              acc[n * R + r] = __builtin_fmaf(df[r], s, acc[n * R + r]);
            }
          }
        }
      }
    }

    int base = 0;
    TeamReduce<VP, MINC, LPR / 2>::run(acc, p, base);
    const bool owner = (p & Shape::OWNER_MASK) == 0;
    epi.template emit<NT, R, Shape::CNT>(rbase, base, owner, acc);
  }
}

}  // namespace q8
