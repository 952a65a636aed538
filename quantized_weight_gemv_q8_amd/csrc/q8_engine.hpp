// q8_engine.hpp -- device core shared by every Q8_0 GEMV kernel (gfx950).
//
// The decode matvec is bound by HBM: each weight byte is used once per
// token, so the kernel's job is to stream the quant and scale planes at the
// memory system's rate and keep everything else off the critical path
// (memra wiki: plain decode is limited by DRAM bandwidth; memra
// performance, the dense IQ4_XS qmatvec table, first arm: wide aligned
// loads relieve the load queue).
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
// result is bitwise identical whatever the batch (memra wiki, gate
// paragraph: K=1..8 speculative verify must equal plain decode, and the
// order of floating-point sums is treated as part of the contract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_format.h"

namespace q8 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 512;  // threads per workgroup for every row kernel
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kOnceMaxBlock = 1024;  // largest workgroup of the one-group-per-wave kernels

// Threads per workgroup of the persistent row kernels. Passes of 4 to 8
// tokens use 12-wave workgroups: the 2 x 17408 x 5120 pair at N = 4 runs
// two per CU (24 waves) in 35.0 us against 38.5 us for three 8-wave ones
// (also 24 waves), and at N = 8 (LDS for one workgroup per CU) 53.2 us
// against 54.9 for two 8-wave ones; 6-, 10- and 16-wave workgroups were
// 10-20% slower (measured on MI355X, same-process A/B). Q4_0 17408 x 5120
// at N = 4: 6% faster.
template <int NT>
constexpr int narrow_block() { return NT >= 4 ? 12 * kWave : kBlock; }

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

// The same 8 fp16 pairs by converting each byte directly: SDWA byte
// selects with sign extension into v_cvt_f16_i16, two instructions per
// pair (the second writes the high half and keeps the low one) against
// five per two pairs above. The values, and so every bit of every result,
// are the same (int8 -> fp16 is exact both ways). Written as asm because
// this compiler shifts each byte down and packs the halves instead of
// using the byte selects and the preserving half write. Used by the
// persistent loop from 4 tokens per pass, where the dot products bound the
// kernel: measured on MI355X (same-process A/B, bitwise equal outputs),
// the 2 x 17408 x 5120 pair at 5-7 tokens 2.6-3.4% faster, the SiLU pair
// at 8 tokens 2.4%, the 151936-row LM head at 4-8 tokens 1.6-2.7%. In
// the one-group kernels the register allocation around the asm blocks
// spilled at 6-8 tokens (4096 x 4096 at 8 tokens 5% slower), so they keep
// the conversion above.
__device__ __forceinline__ void quants_to_h2_sdwa(const uint4 q, h2_t out[8]) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned lo, hi;
    asm("v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "=&v"(lo), "=&v"(hi)
        : "v"(w[i]));
    out[2 * i] = __builtin_bit_cast(h2_t, lo);
    out[2 * i + 1] = __builtin_bit_cast(h2_t, hi);
  }
}

// The first pair of a dot-product chain, a*b summed onto a zero. With ZA
// it is v_dot2_f32_f16 taking the zero as an inline constant; the builtin
// given a zero accumulator becomes a move of 0 plus the two-address v_dot2c
// form, one more VALU op per chain for the same operation (measured on
// MI355X: 3% off the 2 x 17408 x 5120 pair at 4-16 tokens, where the
// dot products bound the kernel; at 1-2 tokens the asm block's scheduling
// barrier costs more than the op, so those kernels keep the builtin).
template <bool ZA>
__device__ __forceinline__ float dot2_from_zero(h2_t a, h2_t b) {
  if constexpr (ZA) {
    float s;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(s) : "v"(a), "v"(b));
    return s;
  } else {
    return __builtin_amdgcn_fdot2(a, b, 0.0f, false);
  }
}

// sum_{i<16} q_i * x_i in fp32, sequential over the 8 pairs in K order.
template <bool ZA>
__device__ __forceinline__ float dot16_f16(const h2_t q[8], const uint4 xlo, const uint4 xhi) {
  float s = dot2_from_zero<ZA>(q[0], __builtin_bit_cast(h2_t, xlo.x));
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

// Weight quants are read exactly once per pass: a non-temporal load
// (global_load_dwordx4 ... nt) keeps them from displacing x, the scales and
// the outputs in the caches. Measured on MI355X: a 151936 x 5120 LM head
// goes from ~143 us to ~124 us (6.6 TB/s) with this hint alone.
__device__ __forceinline__ uint4 load_stream16(const int8_t* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------- weight formats
// A packed row is a sequence of 16-byte chunks. Q8_0: 16 int8 quants per
// chunk, one fp16 scale per 32-quant block (two chunks). Q4_0: one whole
// GGUF block per chunk (16 bytes of 4-bit values stored with +8: the low
// nibble of byte j is element j, the high nibble element j + 16) with its
// own scale. The format decides only the per-chunk dequantisation and the
// scale index; loads, staging, reduction and epilogues are shared.
template <int F>
struct Fmt;
template <>
struct Fmt<kFmtQ8> {
  static constexpr int kElems = 16;      // weights per 16-byte chunk
  static constexpr int kScaleShift = 1;  // scale index = chunk >> shift
};
template <>
struct Fmt<kFmtQ4> {
  static constexpr int kElems = 32;
  static constexpr int kScaleShift = 0;
};

// 16-byte pieces of one row's scales (8 fp16 per piece; a scale row is
// read in whole pieces, which the 8-element row alignment of the scale
// plane keeps in bounds).
__host__ __device__ constexpr int row_scale_pieces(int fmt, int C) {
  return ((fmt == kFmtQ4 ? C : C / 2) + 7) / 8;
}

// 16-byte pieces of x per chunk in the LDS image.
template <int F, bool XF32>
struct ChunkPlanes {
  static constexpr int P = Fmt<F>::kElems * (XF32 ? 4 : 2) / 16;
};

// One Q4_0 block (16 bytes) -> 16 fp16 pairs in element order: pairs 0..7
// from the low nibbles (elements 0..15), 8..15 from the high nibbles. Each
// nibble u = q + 8 is placed under an exponent byte of 0x64 (the fp16 value
// 1024 + u) and 1032 is subtracted: exact, as for the int8 quants.
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
// xs[0..3] hold elements 0-7, 8-15, 16-23 and 24-31.
template <bool ZA>
__device__ __forceinline__ float dot32_f16(const h2_t q[16], const uint4 xs[4]) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = i == 0 ? dot2_from_zero<ZA>(q[0], __builtin_bit_cast(h2_t, xs[0].x))
               : __builtin_amdgcn_fdot2(q[4 * i + 0], __builtin_bit_cast(h2_t, xs[i].x), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 1], __builtin_bit_cast(h2_t, xs[i].y), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 2], __builtin_bit_cast(h2_t, xs[i].z), s, false);
    s = __builtin_amdgcn_fdot2(q[4 * i + 3], __builtin_bit_cast(h2_t, xs[i].w), s, false);
  }
  return s;
}

// fp32 activations: one half of a Q4_0 block (elements 16*half ..
// 16*half + 15: the low nibbles for half 0, the high ones for half 1) as
// exact fp16 values (nibble + 1024 under the 0x64 exponent byte, minus 1032),
// converted once per chunk and row for all tokens.
__device__ __forceinline__ void half_nibbles_to_h2(const uint4 q, int half, h2_t out[8]) {
  const unsigned w[4] = {q.x, q.y, q.z, q.w};
  const h2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned nib = (w[i] >> (4 * half)) & 0x0F0F0F0Fu;
    out[2 * i] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, nib, 0x04010400u)) - bias;
    out[2 * i + 1] =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, nib, 0x04030402u)) - bias;
  }
}

// sum over the 16 elements of that half of q_i * x_i, an fp32 FMA chain in K
// order continuing from s (each fp16 value widens exactly; the FMA is the
// one a converted nibble would take, so the result is bit for bit the same
// as converting each nibble on the spot).
__device__ __forceinline__ float dot16_f32_h(const h2_t w[8], const uint4 x[4], float s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 xv = __builtin_bit_cast(float4, x[i]);
    s = __builtin_fmaf((float)w[2 * i][0], xv.x, s);
    s = __builtin_fmaf((float)w[2 * i][1], xv.y, s);
    s = __builtin_fmaf((float)w[2 * i + 1][0], xv.z, s);
    s = __builtin_fmaf((float)w[2 * i + 1][1], xv.w, s);
  }
  return s;
}

// One chunk c of R rows (quants q[r], fp16 scale bits d[r]) against the LDS
// image xb of the live tokens n < nt: acc[n*R + r] += fp32(d) * chunk sum.
template <int F, int NT, int R, bool XF32, bool SDWA = false>
__device__ __forceinline__ void chunk_fma(const uint4* q, const uint32_t* d, const uint4* xb, int C,
                                          int c, int nt, float* acc) {
  constexpr int P = ChunkPlanes<F, XF32>::P;
  float df[R];
#pragma unroll
  for (int r = 0; r < R; ++r) df[r] = half_bits_to_float((uint16_t)d[r]);
  if constexpr (F == kFmtQ8 && !XF32) {
    h2_t qh[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (SDWA) quants_to_h2_sdwa(q[r], qh[r]);
      else quants_to_h2(q[r], qh[r]);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n >= nt) continue;  // not break: a fixed trip count keeps acc[] in registers
      const uint4 xlo = xb[(n * P + 0) * C + c];
      const uint4 xhi = xb[(n * P + 1) * C + c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sum = dot16_f16<(NT >= 4)>(qh[r], xlo, xhi);
        acc[n * R + r] = __builtin_fmaf(df[r], sum, acc[n * R + r]);
      }
    }
  } else if constexpr (F == kFmtQ8) {
    float qf[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r) quants_to_f32(q[r], qf[r]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n >= nt) continue;  // not break: a fixed trip count keeps acc[] in registers
      const float4 x0 = __builtin_bit_cast(float4, xb[(n * P + 0) * C + c]);
      const float4 x1 = __builtin_bit_cast(float4, xb[(n * P + 1) * C + c]);
      const float4 x2 = __builtin_bit_cast(float4, xb[(n * P + 2) * C + c]);
      const float4 x3 = __builtin_bit_cast(float4, xb[(n * P + 3) * C + c]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sum = dot16_f32(qf[r], x0, x1, x2, x3);
        acc[n * R + r] = __builtin_fmaf(df[r], sum, acc[n * R + r]);
      }
    }
  } else if constexpr (!XF32) {
    h2_t qh[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r) nibbles_to_h2(q[r], qh[r]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n >= nt) continue;  // not break: a fixed trip count keeps acc[] in registers
      uint4 xs[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) xs[h] = xb[(n * P + h) * C + c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sum = dot32_f16<(NT >= 4)>(qh[r], xs);
        acc[n * R + r] = __builtin_fmaf(df[r], sum, acc[n * R + r]);
      }
    }
  } else {
    // Half a block (16 activations) of a token at a time, each (row, token)
    // chain carried across the halves: the same FMA order as one pass over
    // the block, with a quarter of the activation registers live; the half's
    // nibbles are converted once for all tokens.
    float sum[NT][R];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < R; ++r) sum[n][r] = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      h2_t qh[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) half_nibbles_to_h2(q[r], half, qh[r]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n >= nt) continue;  // not break: a fixed trip count keeps acc[] in registers
        uint4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = xb[(n * P + 4 * half + i) * C + c];
#pragma unroll
        for (int r = 0; r < R; ++r) sum[n][r] = dot16_f32_h(qh[r], xv, sum[n][r]);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n >= nt) continue;  // not break: a fixed trip count keeps acc[] in registers
#pragma unroll
      for (int r = 0; r < R; ++r) acc[n * R + r] = __builtin_fmaf(df[r], sum[n][r], acc[n * R + r]);
    }
  }
}

// The one-group kernels that take the SDWA conversion: Q8_0, fp16 x and
// 64-lane rows at 4 or 8 tokens, except the two chunk counts where the
// register allocation around the asm spilled (8 tokens, 4 chunks per lane:
// 4096 x 4096 at N = 8 5% slower) or lost occupancy (4 tokens, 10 chunks).
// Measured on MI355X (same-process A/B, bitwise equal outputs): 5120 x
// 5120 at N = 4 / 8 / 9 / 16 5.0 / 2.8 / 1.9 / 3.2% faster, 4096 x 4096
// and 1024 x 1024 at N = 4 1.0 and 1.4%; 5 to 7 tokens gained nothing.
template <int F, int NT, int LPR, int CPL, bool XF32>
constexpr bool once_sdwa() {
  return F == kFmtQ8 && !XF32 && LPR == 64 && ((NT == 4 && CPL != 10) || (NT == 8 && CPL != 4));
}

// ---------------------------------------------------------------- x staging
// LDS image of x for one pass: token n, plane h (16-byte piece h of a chunk:
// 2 planes for fp16, 4 for fp32), chunk c at uint4 index (n*P + h)*C + c.
template <bool XF32>
struct XPlanes {
  static constexpr int P = XF32 ? 4 : 2;
};

// rows[n] points at token n's K activations (16-byte aligned); rows[0]
// must not be null. Tokens n >= nt, and tokens whose row is null, are not
// staged. Thread t copies pieces t, t + blockDim, ... of every token. The
// loads of a batch (up to 4 tokens x KB pieces) are issued before its LDS
// writes, so staging costs about one memory round trip per batch rather
// than one per token and piece (measured on MI355X: 5120 x 5120 at N = 8
// 19.3 -> 16.8 us). Inside a batch every load is unconditional (a dead
// slot re-reads piece 0 of rows[0] and discards it), so no branch forces a
// wait between the loads; lanes with nothing to copy skip the batch.
template <int NT, int P, int KB>
__device__ __forceinline__ void stage_batch(const char* const rows[NT], int C, uint4* lds, int nt,
                                            int per_tok, int k0) {
  constexpr int TB = NT < 4 ? NT : 4;  // tokens per batch
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const int step = (int)blockDim.x;
  if ((int)threadIdx.x + k0 * step >= per_tok) return;
  const v4u* r0 = reinterpret_cast<const v4u*>(rows[0]);
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += TB) {
    v4u v[TB][KB];
    int dst[TB][KB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int n = n0 + t;
        const int j = (int)threadIdx.x + (k0 + kk) * step;
        const v4u* r = n < NT ? reinterpret_cast<const v4u*>(rows[n < NT ? n : 0]) : nullptr;
        const bool live = n < nt && j < per_tok && r != nullptr;
        v[t][kk] = live ? r[j] : r0[0];
        const int c = j / P, h = j - c * P;
        dst[t][kk] = live ? (n * P + h) * C + c : -1;
      }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
        if (dst[t][kk] >= 0) reinterpret_cast<v4u*>(lds)[dst[t][kk]] = v[t][kk];
    }
  }
}

// KBMAX = 1 keeps the batch (and the kernel's register count) small for
// kernels whose rows need at most one piece per thread and token. P is the
// number of 16-byte pieces of x per chunk (stage_x picks it from the x
// type for 16-quant chunks; other chunk widths call stage_planes).
template <int NT, int P, int KBMAX = 2>
__device__ __forceinline__ void stage_planes(const char* const rows[NT], int C, uint4* lds,
                                             int nt = NT) {
  const int per_tok = C * P;
  if constexpr (NT == 1) {
    // One token: the plain loop measured as fast as batching (2.98 against
    // 3.04 us at 1024 x 1024), with fewer instructions.
    const uint4* src = reinterpret_cast<const uint4*>(rows[0]);
    for (int i = threadIdx.x; i < per_tok; i += blockDim.x) {
      const int c = i / P, h = i - c * P;
      lds[h * C + c] = src[i];
    }
    return;
  }
  const int step = (int)blockDim.x;
  const int kc = (per_tok + step - 1) / step;  // pieces per thread per token
  // The first batch is outside any loop (the only one for K <= 8192 at
  // fp16), so nothing carried around a loop makes its loads wait.
  if (KBMAX == 1 || kc == 1) {
    stage_batch<NT, P, 1>(rows, C, lds, nt, per_tok, 0);
    for (int k0 = 1; k0 < kc; ++k0) stage_batch<NT, P, 1>(rows, C, lds, nt, per_tok, k0);
  } else {
    stage_batch<NT, P, 2>(rows, C, lds, nt, per_tok, 0);
    for (int k0 = 2; k0 < kc; k0 += 2) stage_batch<NT, P, 2>(rows, C, lds, nt, per_tok, k0);
  }
}

template <int NT, bool XF32, int KBMAX = 2>
__device__ __forceinline__ void stage_x(const char* const rows[NT], int C, uint4* lds, int nt = NT) {
  stage_planes<NT, XPlanes<XF32>::P, KBMAX>(rows, C, lds, nt);
}

// The LDS image for chunks of format F (C chunks per row).
template <int F, int NT, bool XF32, int KBMAX = 2>
__device__ __forceinline__ void stage_fmt(const char* const rows[NT], int C, uint4* lds,
                                          int nt = NT) {
  stage_planes<NT, ChunkPlanes<F, XF32>::P, KBMAX>(rows, C, lds, nt);
}

// ---------------------------------------------------------------- staging orders
// A one-group kernel (run_once) calls stage.issue() before its first scale
// or weight load and stage.finish() once the weight loads of its window are
// in flight; finish() leaves the x image in LDS and ends at the workgroup
// barrier.
//
// LateStage: everything in finish() (the image's loads then come after
// the weights, and the barrier after the weights' round trip).
template <class Fn>
struct LateStage {
  Fn fn;
  __device__ __forceinline__ void issue() {}
  __device__ __forceinline__ void finish() { fn(); }
};
template <class Fn>
__device__ __forceinline__ LateStage<Fn> late_stage(Fn fn) {
  return LateStage<Fn>{fn};
}

// EarlyStage: issue() loads this thread's pieces of the x image (XB per
// token, pieces t, t + blockDim, ...) into registers ahead of every weight
// load. Vector memory loads return in issue order, so the image is the
// first data back; finish() writes it to LDS and reaches the barrier while
// the weights are still on their way, instead of after they arrived. The
// loads are unconditional (a piece past the end re-reads the first piece
// and is dropped): no branch, so no wait is forced between them. The LDS
// writes are unconditional too (a dropped piece goes to lds[NT * P * C],
// the first slot past the image, which the caller may reuse only after
// finish()): a conditional write would let the compiler sink the load into
// its branch, behind the weight loads. The launch keeps C * P <= XB *
// blockDim.x. Token n's row starts at x + n * ldx (16-byte aligned).
template <int NT, int P, int XB, bool SYNC = false>
struct EarlyStage {
  const char* x;
  int64_t ldx;  // bytes
  int C;
  int nt;
  uint4* lds;
  uint4 v[NT][XB];
  __device__ __forceinline__ void issue() {
    const int per_tok = C * P;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int k = (int)threadIdx.x + i * (int)blockDim.x;
        const bool live = n < nt && k < per_tok;
        v[n][i] = *reinterpret_cast<const uint4*>(live ? x + n * ldx + 16 * (int64_t)k : x);
      }
    if constexpr (SYNC) __builtin_amdgcn_s_barrier();
  }
  __device__ __forceinline__ void finish() {
    const int per_tok = C * P;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int k = (int)threadIdx.x + i * (int)blockDim.x;
        const int c = k / P, h = k - c * P;
        const bool live = n < nt && k < per_tok;
        lds[live ? (n * P + h) * C + c : NT * P * C] = v[n][i];
      }
    __syncthreads();
  }
};

// ---------------------------------------------------------------- wave maximum
// Maximum of a 64-bit key over the 64 lanes, returned in every lane. DPP
// moves inside each 16-lane row (quad permutes [1,0,3,2] and [2,3,0,1],
// then the half-row and row mirrors) leave every lane with its row's
// maximum; the four row maxima are read with readlane and combined in
// scalar registers. Exact (moves and integer compares only) and about a
// tenth of the latency of a shuffle butterfly through the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = umax64(k, dpp_u64<0xB1>(k));   // quad_perm [1,0,3,2]
  k = umax64(k, dpp_u64<0x4E>(k));   // quad_perm [2,3,0,1]
  k = umax64(k, dpp_u64<0x141>(k));  // row_half_mirror
  k = umax64(k, dpp_u64<0x140>(k));  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 16 * r);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 16 * r);
    m = umax64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
}

// ---------------------------------------------------------------- lane exchange
// The value of lane (lane ^ DELTA), without the LDS crossbar where the
// hardware has a direct path: DPP quad permutes for 1 and 2, ds_swizzle in
// xor mode for 4, 8 and 16 (within 32 lanes), and the gfx950 permlane32
// swap for 32 (each half of the wave reads the other half). Every lane of
// the wave must be active.
template <int DELTA>
__device__ __forceinline__ float xor_lane(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  unsigned r;
  if constexpr (DELTA == 1) {
    r = __builtin_amdgcn_update_dpp(0u, u, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (DELTA == 2) {
    r = __builtin_amdgcn_update_dpp(0u, u, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (DELTA == 4 || DELTA == 8 || DELTA == 16) {
    r = (unsigned)__builtin_amdgcn_ds_swizzle((int)u, 0x1F | (DELTA << 10));
  } else {
    static_assert(DELTA == 32, "xor distance within a wave");
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r = (threadIdx.x & 32) ? sw[0] : sw[1];
  }
  return __builtin_bit_cast(float, r);
}

// v + (the v of lane ^ DELTA), the same bits in both lanes of each pair
// (fp32 addition is commutative).
template <int DELTA>
__device__ __forceinline__ float pair_sum(float v) {
  return v + xor_lane<DELTA>(v);
}

// One halving level over a pair of values (a, b): a lane whose DELTA bit is
// clear returns a + (its partner's a), one whose bit is set b + (its
// partner's b).
// With SW, distances 32 and 16 take one gfx950 half swap of a against b:
// v_permlane32_swap_b32 exchanges the upper 32 lanes of a with the lower 32
// lanes of b, v_permlane16_swap_b32 each odd 16-lane row of a with the even
// row before it in b. Afterwards a first-half lane holds its own a and its
// partner's a, a second-half lane its partner's b and its own b, so the
// sum of the two results is the pair sum with no select. (Swapping a value
// against itself must not take this path: this compiler folds the sum of
// that swap's two results into twice the first, which is why pair_sum
// selects.) Other distances, and every distance without SW, select what
// to send and what to keep around one exchange. Both forms add the same
// two values, so the choice never changes a result.
template <int DELTA, bool SW>
__device__ __forceinline__ float half_sum(float a, float b, bool hi) {
  if constexpr (SW && (DELTA == 16 || DELTA == 32)) {
    const unsigned x = __builtin_bit_cast(unsigned, a), y = __builtin_bit_cast(unsigned, b);
    const auto sw = DELTA == 32 ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                                : __builtin_amdgcn_permlane16_swap(x, y, false, false);
    return __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
  } else {
    const float send = hi ? a : b;
    const float keep = hi ? b : a;
    return keep + xor_lane<DELTA>(send);
  }
}

// ---------------------------------------------------------------- team reduction
// Butterfly over the LPR lanes of a team, xor distances LPR/2, LPR/4, ..., 1.
// While a lane carries more than MINC values, each level halves them
// (the lane keeps the half selected by its distance bit and receives the
// partner's copy of that half), so R*NT sums cost about R*NT shuffles
// instead of log2(LPR) each (the exchanges use half_sum and pair_sum). Every value is
// summed over the same pairing
// tree (partners differing in bit LPR/2, then LPR/4, ...), whatever the
// number of values carried, so the result of each (row, token) does not
// depend on R or NT. fp32 addition is commutative, so the side a value
// arrives from does not matter.
template <int CNT, int MINC, int DELTA, bool SW = false>
struct TeamReduce {
  static __device__ __forceinline__ void run(float* v, int p, int& base) {
    if constexpr (DELTA == 0) {
      return;
    } else if constexpr (CNT > MINC) {
      constexpr int H = CNT / 2;
      const bool hi = (p & DELTA) != 0;
      float nv[H];
#pragma unroll
      for (int i = 0; i < H; ++i) nv[i] = half_sum<DELTA, SW>(v[i], v[i + H], hi);
#pragma unroll
      for (int i = 0; i < H; ++i) v[i] = nv[i];
      if (hi) base += H;
      TeamReduce<H, MINC, DELTA / 2, SW>::run(v, p, base);
    } else {
#pragma unroll
      for (int i = 0; i < CNT; ++i) v[i] = pair_sum<DELTA>(v[i]);
      TeamReduce<CNT, MINC, DELTA / 2, SW>::run(v, p, base);
    }
  }
};

// Where the reduction takes the half swaps: Q8_0 weights, fp16 x and
// 64-lane rows (the large matrices of the decode step). Measured on MI355X
// (same-process A/B, bitwise equal outputs): 1.5-3.5% off 3- to 16-token
// passes of 5120 x 5120 and of the 2 x 17408 x 5120 pair and SiLU pair,
// 1.5% off the router; the 151936-row LM head at 8 tokens 2% slower.
// Elsewhere the register allocation that follows cost occupancy or
// spilled (Q4_0 and fp32-x one-group kernels at 5-7 tokens), so those keep
// the selects.
template <int F, int LPR, bool XF32>
constexpr bool swap_reduce() { return F == kFmtQ8 && !XF32 && LPR == 64; }

// Waves per SIMD the register budget of a persistent row kernel must
// allow: six for 4-token passes with the half swaps, so that two 12-wave
// workgroups share a CU as the LDS allows (the swaps' register allocation
// would otherwise take 86 registers and leave room for one); otherwise no
// bound beyond the workgroup's own.
template <int F, int NT, int LPR, bool XF32>
constexpr int narrow_waves_per_simd() { return NT == 4 && swap_reduce<F, LPR, XF32>() ? 6 : 1; }

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

// Rows per team (R) and load-window depth in chunks (D) per token count
// and size class. R rows share each LDS read of x (LDS bytes per weight
// byte = 2*NT/R for fp16 x); D*R 16-byte loads are kept in flight per wave.
// Neither changes the per-(row, token) arithmetic, so the choice may depend
// on the shape (per-shape dispatch) without breaking N-invariance.
// Measured on MI355X (persistent grid at full occupancy, same-process A/B):
// a one-chunk window (D = 1) with many resident waves beats deeper windows
// at every width; at N = 1 large matrices (>= 64K rows, e.g. a 151936-row
// LM head) stream best with R = 4 and smaller ones with R = 1; for N >= 3,
// R = 4 keeps the LDS reads of x per weight byte low.
template <int NT, bool BIG>
struct Tune {
  static constexpr int R = NT == 1 ? (BIG ? 4 : 1) : (NT <= 2 ? 2 : 4);
  static constexpr int D = 1;
};
constexpr int64_t kBigRows = 65536;

// Shape modes of the dense GEMV: 0 as Tune<NT, false>, 1 as Tune<NT, true>
// (>= 64K rows at N = 1), 2 for matrices too small to give every CU a row
// group (a router, a small projection): one row per team and two chunk
// loads in flight, so the few waves there are each issue their whole row
// at once. R and D never change the arithmetic of a (row, token).
template <int NT, int MODE>
struct TuneM {
  static constexpr int R = MODE == 2 ? 1 : Tune<NT, MODE == 1>::R;
  static constexpr int D = MODE == 2 ? 2 : Tune<NT, MODE == 1>::D;
};

// ---------------------------------------------------------------- row sources
struct MatDesc {
  const int8_t* qs;
  const uint16_t* d;
  int64_t ld_qs;  // bytes
  int64_t ld_d;   // fp16 elements
};

// ---------------------------------------------------------------- engine
// A wave walks the (group, chunk) iterations of the groups g = g_first,
// g_first + g_stride, ... < n_groups, chunk j = 0..CPL-1 inside a group.
// Loads run D iterations ahead of the arithmetic in a ring of D register
// slots, across group boundaries, so each wave keeps D*R 16-byte quant
// loads (plus their scales) in flight at all times, and the first D are
// issued before x is staged (the caller's `stage`, which ends with a
// workgroup barrier). The iteration count is padded to a multiple of D;
// padded iterations load nothing and emit nothing.
//
// map.row(i, q, d) gives row i's planes (false if row i does not exist or is
// outside the caller's tile). epi.emit(row_base, base, owner, v) receives
// the reduced sums of one group: values v[0..CNT) are (token n, row r)
// pairs with flat index base+i = n*R + r, rows row_base + r.
template <int R>
struct Slot {
  uint4 q[R];
  uint32_t d[R];
};

// nt <= NT is the number of live tokens (wave-uniform); tokens n >= nt are
// skipped, so one instantiation serves any count up to NT with the same
// per-token arithmetic.
template <int NT, int LPR, int R, int D, int MINC, bool XF32, int F = kFmtQ8, class Map, class Epi,
          class Stage>
__device__ __forceinline__ void run_rows(const Map& map, Epi& epi, const uint4* lds, int C,
                                         int64_t n_groups, int64_t g_first, int64_t g_stride,
                                         int64_t row_origin, Stage&& stage, int nt = NT) {
  constexpr int RPW = kWave / LPR;  // teams per wave
  constexpr int G = RPW * R;        // rows per wave per group
  constexpr int V = NT * R;
  constexpr int VP = Pow2<V>::value;
  using Shape = ReduceShape<LPR, VP, MINC>;

  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane % LPR;
  const int team = lane / LPR;
  const int CPL = (C + LPR - 1) / LPR;

  // Groups of this wave. The callers' g_first and g_stride are wave-uniform,
  // so this is scalar code; a 32-bit quotient keeps it short in front of
  // the first load (a 64-bit division is a long instruction sequence).
  int64_t my_groups = 0;
  if (g_first < n_groups) {
    const int64_t num = n_groups - g_first + g_stride - 1;
    my_groups = num <= (int64_t)UINT32_MAX ? (int64_t)((uint32_t)num / (uint32_t)g_stride)
                                           : num / g_stride;
  }
  const int64_t total = my_groups * CPL;
  const int64_t padded = (total + D - 1) / D * D;

  Slot<R> slot[D];
  int64_t ig = g_first;  // issue cursor: group and chunk
  int ij = 0;
  // Row pointers of the issue cursor's group, refreshed once per group: the
  // per-chunk issue is then one add, which keeps the load-to-next-load path
  // short when only a few loads per wave are in flight.
  const int8_t* iq[R];
  const uint16_t* id[R];
  bool iok[R];
  auto refresh = [&]() {
    const bool live = ig < n_groups;
    const int64_t rbase = row_origin + ig * G + (int64_t)team * R;
#pragma unroll
    for (int r = 0; r < R; ++r) iok[r] = live && map.row(rbase + r, iq[r], id[r]);
  };
  refresh();
  auto issue = [&](Slot<R>& sl) {
    const int c = p + LPR * ij;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (iok[r] && c < C) {
        sl.q[r] = load_stream16(iq[r] + (int64_t)c * 16);
        sl.d[r] = id[r][c >> Fmt<F>::kScaleShift];
      } else {
        sl.q[r] = make_uint4(0, 0, 0, 0);
        sl.d[r] = 0;
      }
    }
    if (++ij == CPL) {
      ij = 0;
      ig += g_stride;
      refresh();
    }
  };

#pragma unroll
  for (int s = 0; s < D; ++s) issue(slot[s]);
  stage();

  float acc[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
  int64_t cg = g_first;
  int cj = 0;

  for (int64_t it = 0; it < padded; it += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int c = p + LPR * cj;
      if (c < C) chunk_fma<F, NT, R, XF32, (NT >= 4)>(slot[s].q, slot[s].d, lds, C, c, nt, acc);
      issue(slot[s]);
      if (++cj == CPL) {
        {
          // No branch on cg here either (see run_once): past the last
          // group the owner flag is false and nothing is emitted.
          int base = 0;
          TeamReduce<VP, MINC, LPR / 2, swap_reduce<F, LPR, XF32>()>::run(acc, p, base);
          const bool owner = (p & Shape::OWNER_MASK) == 0 && cg < n_groups;
          const int64_t rbase = row_origin + cg * G + (int64_t)team * R;
          epi.template emit<NT, R, Shape::CNT>(rbase, base, owner, acc);
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
        cj = 0;
        cg += g_stride;
      }
    }
  }
}

// One row group per wave, C = CPL * LPR chunks per row known at compile
// time. The chunk loop is written out, with loads D chunks ahead of the
// arithmetic, so the compiler sees every load and every wait statically
// and may schedule the loads earlier still; there is no group loop, no
// cursor and no padding. Rows past last_row read last_row (their values are
// never emitted), so every load is unconditional. A wave with g >= n_groups
// loads and stages like the others (the workgroup barrier in stage() needs
// every wave) and emits nothing. Per (row, token) the arithmetic is that of
// run_rows: the same chunk order per lane, the same fma and the same
// reduction tree, so results are bitwise those of run_rows.
//
// Scales: the team fetches each of its rows' whole scale row with 16-byte
// loads (once_scale_pieces pieces, lane p takes pieces p, p + LPR, ...),
// issued before the first weight load, and writes it after stage.finish()
// to the wave's own LDS area lds_s + wave * G * pieces (no barrier: only
// this wave reads it); every chunk then reads its scale from LDS. One or
// two loads per row instead of one 2-byte load per chunk. lds_s holds
// waves-per-workgroup * G * once_scale_pieces(F, CPL * LPR) pieces.
// Order of the loads: stage.issue() (x, for an EarlyStage), the scale rows,
// then the first D weight chunks.
template <int NT, int LPR, int R, int CPL, int D, int MINC, bool XF32, int F, class Map, class Epi,
          class Stage>
__device__ __forceinline__ void run_once(const Map& map, Epi& epi, const uint4* lds,
                                         uint4* lds_s, int64_t n_groups, int64_t g,
                                         int64_t row_origin, int64_t last_row, Stage& stage,
                                         int nt = NT) {
  constexpr int RPW = kWave / LPR;
  constexpr int G = RPW * R;
  constexpr int V = NT * R;
  constexpr int VP = Pow2<V>::value;
  constexpr int C = CPL * LPR;
  constexpr int SP = row_scale_pieces(F, C);  // 16-byte pieces of a scale row
  constexpr int NSP = (SP + LPR - 1) / LPR;   // of them per lane
  using Shape = ReduceShape<LPR, VP, MINC>;
  static_assert(D >= 1 && D <= CPL, "window within the row");

  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane % LPR;
  const int team = lane / LPR;
  const int64_t rbase = row_origin + g * G + (int64_t)team * R;
  const int8_t* q[R];
  const uint16_t* d[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = rbase + r;
    map.row(i < last_row ? i : last_row, q[r], d[r]);
  }
  stage.issue();
  // Keep the issue order (x, scales, weights): loads return in that order,
  // and the scheduler would otherwise interleave them freely.
  __builtin_amdgcn_sched_barrier(0);
  // Scale rows: unconditional loads, lanes past the last piece re-read it
  // (same line, no extra traffic).
  uint4 srow[R][NSP];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int k = 0; k < NSP; ++k) {
      const int piece = p + LPR * k;
      srow[r][k] = load_stream16(reinterpret_cast<const int8_t*>(d[r]) +
                                 16 * (piece < SP ? piece : SP - 1));
    }
  __builtin_amdgcn_sched_barrier(0);
  Slot<R> slot[D];
  auto issue = [&](Slot<R>& sl, int j) {
    const int c = p + LPR * j;
#pragma unroll
    for (int r = 0; r < R; ++r) sl.q[r] = load_stream16(q[r] + (int64_t)c * 16);
  };
  // The window's loads in chunk order (each wait below then covers only the
  // chunks before the one it needs).
#pragma unroll
  for (int s = 0; s < D; ++s) {
    issue(slot[s], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage.finish();
  uint4* const srow_lds = lds_s + ((int)(threadIdx.x / kWave) * G + team * R) * SP;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int k = 0; k < NSP; ++k)
      if (p + LPR * k < SP) srow_lds[r * SP + p + LPR * k] = srow[r][k];

  float acc[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = p + LPR * j;
    uint32_t dd[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      dd[r] = reinterpret_cast<const uint16_t*>(srow_lds + r * SP)[c >> Fmt<F>::kScaleShift];
    chunk_fma<F, NT, R, XF32, once_sdwa<F, NT, LPR, CPL, XF32>()>(slot[j % D].q, dd, lds, C, c, nt, acc);
    if (j + D < CPL) issue(slot[j % D], j + D);
  }
  // Reduced and emitted without a branch on g: a wave-uniform early exit
  // here made the compiler restructure the whole kernel around it (about
  // 5% slower at 5120 x 5120); a dead wave's owner flag is simply false.
  int base = 0;
  TeamReduce<VP, MINC, LPR / 2, swap_reduce<F, LPR, XF32>()>::run(acc, p, base);
  const bool owner = (p & Shape::OWNER_MASK) == 0 && g < n_groups;
  epi.template emit<NT, R, Shape::CNT>(rbase, base, owner, acc);
}

}  // namespace q8
