// q8_router.hip -- the router of a routed layer on the device (gfx950).
//
// The pages keep routing on the device, as graph-replayable device-side
// lengths and counters (memra wiki, feature list), and route with
// m-invariant kernels so that a token's experts never depend on the other
// tokens of the batch (memra performance, serving exactness arc). Per
// token: the topk experts with the largest router logits (descending,
// equal logits to the lower expert index, -0 equal to +0) and softmax
// weights over the picked logits. One wave owns one token, so a token's
// result cannot depend on the batch. From a Q8_0 router matrix, 9 to 64
// tokens run as one launch (router_kernel: one workgroup per token, the
// logits kept in LDS); other shapes take the GEMV, then topk_softmax_kernel.
//
// Selection: every logit becomes a 64-bit key, (order-preserving bits of
// the fp32 value) << 32 | ~expert, so the largest key is the largest
// logit and, among equal logits, the lowest expert. Each lane keeps the
// keys of its own experts (expert e belongs to lane e % 64); a pick is a
// wave maximum, after which the owner of the picked expert drops it: up to
// 256 experts the keys stay in registers, beyond that the owner rescans
// its (at most 64) experts from LDS. The wave maximum runs on DPP moves
// and readlanes (wave_max_u64), not on shuffles through the LDS crossbar.
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

__device__ __forceinline__ uint32_t router_ord(float v) {
  if (v == 0.0f) v = 0.0f;  // -0 -> +0
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float router_value(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ uint64_t router_key(uint32_t o, int e) {
  return ((uint64_t)o << 32) | (uint64_t)(~(uint32_t)e);
}

// Softmax over the picked logits (lane j holds the j-th, the first is the
// largest). The butterfly gives every lane the same sum (each level adds
// the same two numbers on both partners).
__device__ __forceinline__ void softmax_picks(float mine, int topk, int64_t t, float* gate_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const float top = __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(unsigned, mine), 0));
  const float z = lane < topk ? expf(mine - top) : 0.0f;
  float s = z;
  s = pair_sum<32>(s);
  s = pair_sum<16>(s);
  s = pair_sum<8>(s);
  s = pair_sum<4>(s);
  s = pair_sum<2>(s);
  s = pair_sum<1>(s);
  if (lane < topk) gate_w[t * topk + lane] = z / s;
}

// Top-k and softmax of token t's logits row[0..E) by one wave (every lane
// active); ord is E uint32 of LDS.
__device__ __forceinline__ void topk_softmax_wave(const float* row, int E, int topk, int64_t t,
                                                  int32_t* ids, float* gate_w, uint32_t* ord) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t best = 0;
  for (int e = lane; e < E; e += kWave) {
    const uint32_t o = router_ord(row[e]);
    ord[e] = o;
    const uint64_t k = router_key(o, e);
    best = k > best ? k : best;
  }
  uint64_t taken = 0;  // bit i: this lane's expert lane + 64 i has been picked
  float mine = 0.0f;   // lane j holds the j-th picked logit
  for (int j = 0; j < topk; ++j) {
    const uint64_t m = wave_max_u64(best);
    const int e = (int)(~(uint32_t)m);
    if (lane == j) mine = router_value((uint32_t)(m >> 32));
    if (lane == 0) ids[(int64_t)t * topk + j] = e;
    if (e % kWave == lane) {
      taken |= 1ull << (e / kWave);
      best = 0;
      for (int i = 0, f = lane; f < E; ++i, f += kWave) {
        if ((taken >> i) & 1ull) continue;
        const uint64_t k = router_key(ord[f], f);
        best = k > best ? k : best;
      }
    }
  }
  softmax_picks(mine, topk, t, gate_w);
}

// The same picks with every candidate key in registers (E <= 64 * KPL):
// after a pick the owner clears that key instead of rescanning LDS. Keys
// are unique (they carry the expert), so the picks are those above.
template <int KPL>
__device__ __forceinline__ void topk_softmax_wave_regs(const float* row, int E, int topk,
                                                       int64_t t, int32_t* ids, float* gate_w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? router_key(router_ord(row[e]), e) : 0;
  }
  float mine = 0.0f;  // lane j holds the j-th picked logit
  for (int j = 0; j < topk; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t m = wave_max_u64(best);
    if (lane == j) mine = router_value((uint32_t)(m >> 32));
    if (lane == 0) ids[t * topk + j] = (int)(~(uint32_t)m);
#pragma unroll
    for (int i = 0; i < KPL; ++i) key[i] = key[i] == m ? 0 : key[i];
  }
  softmax_picks(mine, topk, t, gate_w);
}


// Up to 256 experts the keys stay in registers (same picks, no LDS
// rescans); beyond, in LDS.
__global__ __launch_bounds__(kWave) void topk_softmax_kernel(const float* logits, int E, int topk,
                                                             int32_t* ids, float* gate_w) {
  extern __shared__ uint32_t ord[];  // [E]
  const int64_t t = blockIdx.x;
  const float* row = logits + t * E;
  if (E <= kWave) topk_softmax_wave_regs<1>(row, E, topk, t, ids, gate_w);
  else if (E <= 2 * kWave) topk_softmax_wave_regs<2>(row, E, topk, t, ids, gate_w);
  else if (E <= 4 * kWave) topk_softmax_wave_regs<4>(row, E, topk, t, ids, gate_w);
  else topk_softmax_wave(row, E, topk, t, ids, gate_w, ord);
}

// ---------------------------------------------------------------- fused router
// The whole router in one launch, one workgroup per token: the token's x
// is staged, the one-group engine computes the E logits (the dense GEMV's
// per-row arithmetic, so they are bitwise q8_gemv's) into LDS and to
// `logits`, and one wave takes the top-k and softmax from them. Every wave
// owns one group of RR rows per team and issues all of its loads before x
// is staged, so the matrix streams in one memory round trip; the logits
// never round-trip through memory between launches. One workgroup streams
// the whole matrix, which one compute unit does at a fraction of the chip's
// rate (about 10 us for 128 x 2048, whatever the token count), so it pays
// only where the GEMV would take two or more passes of 8 tokens. Measured
// on MI355X against GEMV + top-k launches (us): 128 x 2048, T = 1 7.2
// against 10.3 (so not taken), T = 16 14.2 -> 10.5, T = 64 41.4 -> 10.7.
// Taken for kRouterFusedMinT..kRouterFusedMaxT tokens, Q8_0 matrices, fp16
// x, E <= kRouterMaxFusedE and at most 16 waves of at most 16 loads per
// lane; otherwise the GEMV and top-k launches run.
constexpr int kRouterMaxFusedE = 4 * kWave;
constexpr int kRouterMaxWaves = 16;
constexpr int kRouterMaxLoads = 16;  // RR * CPL 16-byte loads per lane

struct RouterMap {
  MatDesc w;
  int64_t E;
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    q = w.qs + i * w.ld_qs;
    d = w.d + i * w.ld_d;
    return i < E;
  }
};

struct RouterEpi {
  float* out;  // logits row of this token
  float* lds;  // the same values in LDS
  int64_t E;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int64_t row = rbase + (idx - (idx / R) * R);
      if (row >= E) continue;
      out[row] = v[i];
      lds[row] = v[i];
    }
  }
};

template <int LPR, int CPL, int RR>
__global__ __launch_bounds__(kRouterMaxWaves * kWave) void router_kernel(
    RouterMap map, const char* x, int64_t ldx_bytes, int topk, float* logits, int32_t* ids,
    float* gate_w) {
  extern __shared__ uint4 lds_x[];
  constexpr int F = kFmtQ8;
  constexpr int C = CPL * LPR;
  constexpr int G = (kWave / LPR) * RR;
  constexpr int P = ChunkPlanes<F, false>::P;
  const int64_t t = blockIdx.x;
  const int E = (int)map.E;
  const int waves = (int)(blockDim.x / kWave);
  uint4* lds_s = lds_x + C * P;
  float* lds_logits = reinterpret_cast<float*>(lds_s + waves * G * row_scale_pieces(F, C));
  RouterEpi epi;
  epi.out = logits + t * E;
  epi.lds = lds_logits;
  epi.E = E;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  auto stage = late_stage([=]() {
    const char* rows[1] = {x + t * ldx_bytes};
    stage_fmt<F, 1, false>(rows, C, lds_x);
    __syncthreads();
  });
  run_once<1, LPR, RR, CPL, CPL, 1, false, F>(map, epi, lds_x, lds_s, (E + G - 1) / G, wave, 0,
                                               E - 1, stage);
  __syncthreads();
  if (wave == 0) {
    if (E <= kWave) topk_softmax_wave_regs<1>(lds_logits, E, topk, t, ids, gate_w);
    else if (E <= 2 * kWave) topk_softmax_wave_regs<2>(lds_logits, E, topk, t, ids, gate_w);
    else topk_softmax_wave_regs<4>(lds_logits, E, topk, t, ids, gate_w);
  }
}

template <int LPR, int CPL, int RR>
static hipError_t router_launch_t(const DevInfo& dev, const RouterMap& map, const char* x,
                                  int64_t ldx_bytes, int T, int topk, float* logits, int32_t* ids,
                                  float* gate_w, hipStream_t s) {
  constexpr int G = (kWave / LPR) * RR;
  const int waves = (int)((map.E + G - 1) / G);
  const size_t lds = (size_t)CPL * LPR * 16 * ChunkPlanes<kFmtQ8, false>::P +
                     (size_t)waves * G * row_scale_pieces(kFmtQ8, CPL * LPR) * 16 +
                     (size_t)map.E * 4;
  if (waves > kRouterMaxWaves || lds > dev.lds_per_block) return hipErrorNotSupported;
  const void* fn = (const void*)router_kernel<LPR, CPL, RR>;
  if (hipError_t e = allow_dynamic_lds(fn, lds)) return e;
  void* args[] = {(void*)&map, (void*)&x, &ldx_bytes, &topk, &logits, &ids, &gate_w};
  return hipLaunchKernel(fn, dim3((unsigned)T), dim3(waves * kWave), args, lds, s);
}

// Rows per team: the fewest that fit the rows in kRouterMaxWaves waves.
template <int LPR, int CPL>
static hipError_t router_launch_rr(const DevInfo& dev, const RouterMap& map, const char* x,
                                   int64_t ldx_bytes, int T, int topk, float* logits,
                                   int32_t* ids, float* gate_w, hipStream_t s) {
  const int64_t per_team = (map.E + kRouterMaxWaves * (kWave / LPR) - 1) /
                           (kRouterMaxWaves * (kWave / LPR));
#define Q8_RR(RRV)                                                                              \
  if (per_team <= RRV) {                                                                        \
    if constexpr (RRV * CPL <= kRouterMaxLoads)                                                 \
      return router_launch_t<LPR, CPL, RRV>(dev, map, x, ldx_bytes, T, topk, logits, ids,      \
                                            gate_w, s);                                         \
    return hipErrorNotSupported;                                                                \
  }
  Q8_RR(1) Q8_RR(2) Q8_RR(4) Q8_RR(8)
#undef Q8_RR
  return hipErrorNotSupported;
}

hipError_t launch_router(const DevInfo& dev, const HMat& Wr, const void* x, bool x_f32, int T,
                         int topk, float* logits, int32_t* ids, float* gate_w, hipStream_t s) {
  if (T < kRouterFusedMinT || T > kRouterFusedMaxT || x_f32 || Wr.fmt != kFmtQ8 ||
      Wr.M > kRouterMaxFusedE)
    return hipErrorNotSupported;
  RouterMap map;
  map.w = MatDesc{Wr.qs, Wr.d, Wr.ld_qs, Wr.ld_d};
  map.E = Wr.M;
  const int C = (int)chunks_per_row(Wr.fmt, Wr.K);
  const int lpr = lanes_for(Wr.fmt, Wr.K);
  if (C % lpr != 0) return hipErrorNotSupported;
  const char* xp = (const char*)x;
  const int64_t ldx_bytes = Wr.K * 2;
  auto by_cpl = [&](auto l) -> hipError_t {
    constexpr int L = decltype(l)::value;
    switch (C / L) {
      case 1: return router_launch_rr<L, 1>(dev, map, xp, ldx_bytes, T, topk, logits, ids, gate_w, s);
      case 2: return router_launch_rr<L, 2>(dev, map, xp, ldx_bytes, T, topk, logits, ids, gate_w, s);
      case 4: return router_launch_rr<L, 4>(dev, map, xp, ldx_bytes, T, topk, logits, ids, gate_w, s);
    }
    return hipErrorNotSupported;
  };
  if (lpr == 64) return by_cpl(std::integral_constant<int, 64>{});
  if (lpr == 32) return by_cpl(std::integral_constant<int, 32>{});
  return by_cpl(std::integral_constant<int, 16>{});
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int topk, int32_t* ids,
                               float* gate_w, hipStream_t s) {
  void* args[] = {(void*)&logits, &E, &topk, &ids, &gate_w};
  return hipLaunchKernel((const void*)topk_softmax_kernel, dim3((unsigned)T), dim3(kWave), args,
                         (size_t)E * sizeof(uint32_t), s);
}

}  // namespace q8
