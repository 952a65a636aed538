// q8_router.hip -- the router of a routed layer on the device (gfx950).
//
// The pages keep routing on the device, as graph-replayable device-side
// lengths and counters (memra wiki, feature list), and route with
// m-invariant kernels so that a token's experts never depend on the other
// tokens of the batch (memra performance, serving exactness arc). Per
// token: the topk experts with the largest router logits (descending,
// equal logits to the lower expert index, -0 equal to +0) and softmax
// weights over the picked logits. One wave owns one token, so a token's
// result cannot depend on the batch.
//
// Selection: every logit becomes a 64-bit key, (order-preserving bits of
// the fp32 value) << 32 | ~expert, so the largest key is the largest
// logit and, among equal logits, the lowest expert. Each lane keeps the
// best key of its own experts (expert e belongs to lane e % 64); a pick is
// a wave maximum, after which only the owner of the picked expert rescans
// its (at most 64) experts. The wave maximum runs on DPP moves and
// readlanes (wave_max_u64), not on shuffles through the LDS crossbar.
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

__global__ __launch_bounds__(kWave) void topk_softmax_kernel(const float* logits, int E, int topk,
                                                             int32_t* ids, float* gate_w) {
  extern __shared__ uint32_t ord[];  // [E]
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* row = logits + (int64_t)t * E;
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
  // Softmax over the picked logits; the first pick is the largest. The
  // butterfly gives every lane the same sum (each level adds the same two
  // numbers on both partners).
  const float top = __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(unsigned, mine), 0));
  const float z = lane < topk ? expf(mine - top) : 0.0f;
  float s = z;
  s += xor_lane<32>(s);
  s += xor_lane<16>(s);
  s += xor_lane<8>(s);
  s += xor_lane<4>(s);
  s += xor_lane<2>(s);
  s += xor_lane<1>(s);
  if (lane < topk) gate_w[(int64_t)t * topk + lane] = z / s;
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int topk, int32_t* ids,
                               float* gate_w, hipStream_t s) {
  void* args[] = {(void*)&logits, &E, &topk, &ids, &gate_w};
  return hipLaunchKernel((const void*)topk_softmax_kernel, dim3((unsigned)T), dim3(kWave), args,
                         (size_t)E * sizeof(uint32_t), s);
}

}  // namespace q8
