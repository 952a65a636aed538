// q8_router.hip -- the router of a routed layer on the device (gfx950).
//
// The pages keep routing on the device, as graph-replayable device-side
// lengths and counters (memra wiki, feature list), and route with
// m-invariant kernels so that a token's experts never depend on the other
// tokens of the batch (memra performance, serving exactness arc). Per
// token: the topk experts with the largest router logits (descending,
// equal logits to the lower expert index, -0 equal to +0) and softmax
// weights over the picked logits. One wave owns one token, so a token's
// result cannot depend on the batch. From a router matrix the logits come
// from the GEMV, then topk_softmax_kernel picks from them. (A one-launch
// router, one workgroup per token streaming the whole matrix with the
// logits kept in LDS, took about 10.5 us for 128 x 2048 at any token
// count; since the GEMV runs all its passes of 8 tokens in one launch, the
// two launches take 8.2 us at 16-64 tokens and 10.2 at 9, so it was
// removed.)
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

hipError_t launch_topk_softmax(const float* logits, int T, int E, int topk, int32_t* ids,
                               float* gate_w, hipStream_t s) {
  void* args[] = {(void*)&logits, &E, &topk, &ids, &gate_w};
  return hipLaunchKernel((const void*)topk_softmax_kernel, dim3((unsigned)T), dim3(kWave), args,
                         (size_t)E * sizeof(uint32_t), s);
}

}  // namespace q8
