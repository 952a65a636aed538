// q8_lmhead.hip -- LM-head Q8_0 GEMV fused with a greedy argmax (gfx950).
//
// The decode step ends with the vocabulary projection and a greedy pick;
// the pages keep the logits lean and move 4 bytes per token to the host
// (memra wiki, feature list: "CUDA-graph decode ... 4 bytes/token host
// traffic"), and greedy argmax is their correctness instrument (memra wiki,
// gate paragraph: run-gen prints its argmax gate before any number).
//
// Pass structure: one persistent GEMV launch. Each workgroup folds the
// rows it produced into one 64-bit key per token, merges it into a
// per-token slot with an atomic maximum, and then takes a ticket from a
// wrapping counter; the workgroup that draws the last ticket reads the
// slots (resetting them to zero) and decodes the row indices. Slots and
// counter are zero again after every completed launch, so the workspace
// needs zero-filling only before its first use. Key = (order-preserving
// bits of the fp32 logit, with -0 mapped to +0) << 32 | ~row, so the
// maximum key is the largest logit and, among equal logits, the lowest
// row; the result does not depend on the order of the workgroups. A draft
// head (a packed subset of the vocabulary rows) reports the winner through
// its row-id table.
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

constexpr int kLmMaxBlocks = 4096;

__device__ __forceinline__ uint64_t argmax_key(float v, int64_t row) {
  if (v == 0.0f) v = 0.0f;  // -0 -> +0
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(~(uint32_t)row);
}

struct LmMap {
  MatDesc w;
  int64_t V;
  const int32_t* row_ids;  // null, or the vocabulary id of each row (a draft head's subset)
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    q = w.qs + i * w.ld_qs;
    d = w.d + i * w.ld_d;
    return i < V;
  }
};

// Workspace (zero before first use, zero again after every launch):
// per-group slots [kLmGroups][kMaxNT] uint64 and counters, one 256-byte
// line each, then the final slots [kMaxNT] and counter.
constexpr int kLmGroups = 8;
constexpr int kLmLine = 256;
constexpr size_t kLmWsBytes = (size_t)(2 * kLmGroups + 2) * kLmLine;
static_assert(kMaxNT * sizeof(uint64_t) <= kLmLine, "slots fit a line");

struct LmWs {
  char* base;
  __device__ __forceinline__ uint64_t* group_slot(uint32_t g) const {
    return (uint64_t*)(base + (size_t)g * kLmLine);
  }
  __device__ __forceinline__ uint32_t* group_ctr(uint32_t g) const {
    return (uint32_t*)(base + (size_t)(kLmGroups + g) * kLmLine);
  }
  uint64_t* slot;
  uint32_t* ctr;
};

__device__ __forceinline__ LmWs lm_ws(char* ws) {
  LmWs w;
  w.base = ws;
  w.slot = (uint64_t*)(ws + (size_t)(2 * kLmGroups) * kLmLine);
  w.ctr = (uint32_t*)(ws + (size_t)(2 * kLmGroups + 1) * kLmLine);
  return w;
}

// Each lane owns a fixed set of (token, row-slot) values after the team
// reduction (the set depends only on the lane's position), so the running
// best is kept per value slot, indexed at compile time.
template <int CNT>
struct LmEpi {
  float* logits;
  int64_t ld;
  int64_t V;
  float bv[CNT];
  int64_t bi[CNT];
  int my_base;
  bool my_owner;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < CNT; ++i) { bv[i] = 0.0f; bi[i] = -1; }
    my_base = 0;
    my_owner = false;
  }

  template <int NT, int R, int CNT_>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    static_assert(CNT_ == CNT, "slot count");
    // Ownership and base depend only on the lane's position; a call with
    // owner false (a lane that owns nothing, or a group past the end)
    // leaves them and the running best as they are.
    if (!owner) return;
    my_base = base;
    my_owner = true;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (row >= V) continue;
      const float val = v[i];
      if (logits) logits[n * ld + row] = val;
      if (bi[i] < 0 || val > bv[i] || (val == bv[i] && row < bi[i])) {
        bv[i] = val;
        bi[i] = row;
      }
    }
  }
};

template <int F, int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(kBlock) void lmhead_kernel(LmMap map, float* logits, int64_t ld,
                                                        const char* x, int64_t ldx_bytes, int C,
                                                        char* ws, int32_t* ids) {
  extern __shared__ uint4 lds_x[];
  __shared__ uint64_t red[kWavesPerBlock][kMaxNT];
  using T = Tune<NT, BIG>;
  constexpr int R = T::R;
  constexpr int G = (kWave / LPR) * R;
  constexpr int VP = Pow2<NT * R>::value;
  constexpr int CNT = ReduceShape<LPR, VP, 1>::CNT;

  LmEpi<CNT> epi;
  epi.logits = logits;
  epi.ld = ld;
  epi.V = map.V;
  epi.init();
  const int64_t n_groups = (map.V + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
    stage_fmt<F, NT, XF32>(rows, C, lds_x);
    __syncthreads();
  };
  run_rows<NT, LPR, R, T::D, 1, XF32, F>(map, epi, lds_x, C, n_groups,
                                         (int64_t)blockIdx.x * kWavesPerBlock + wave,
                                         (int64_t)gridDim.x * kWavesPerBlock, 0, stage);

#pragma unroll
  for (int n = 0; n < NT; ++n) {
    uint64_t k = 0;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = epi.my_base + i;
      if (epi.my_owner && idx < NT * R && idx / R == n && epi.bi[i] >= 0) {
        const uint64_t c = argmax_key(epi.bv[i], epi.bi[i]);
        k = c > k ? c : k;
      }
    }
    k = wave_max_u64(k);
    if (lane == 0) red[wave][n] = k;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // Two-level merge of the per-workgroup keys: workgroup b belongs to
    // group b % ng. Every access to the slots and counters is an
    // agent-scope atomic, so each location is coherent across the chip
    // without cache write-back or invalidation, and waiting for the
    // returned values puts a workgroup's slot updates before its ticket.
    const LmWs w = lm_ws(ws);
    const uint32_t ng = gridDim.x < (uint32_t)kLmGroups ? gridDim.x : (uint32_t)kLmGroups;
    const uint32_t g = blockIdx.x % ng;
    const uint32_t members = (gridDim.x - g + ng - 1) / ng;
    uint64_t dep = 0;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      uint64_t k = 0;
      for (int wv = 0; wv < kWavesPerBlock; ++wv) {
        const uint64_t o = red[wv][n];
        k = o > k ? o : k;
      }
      dep |= __hip_atomic_fetch_max(w.group_slot(g) + n, k, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : "v"(dep) : "memory");
    // A counter returns to zero when its last ticket is drawn.
    bool last = atomicInc(w.group_ctr(g), members - 1) == members - 1;
    if (last) {
      // Every member of the group has merged: move the group's keys into
      // the final slots (leaving the group slots at zero).
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint64_t m = __hip_atomic_exchange(w.group_slot(g) + n, (uint64_t)0,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dep |= __hip_atomic_fetch_max(w.slot + n, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      asm volatile("s_waitcnt vmcnt(0)" : : "v"(dep) : "memory");
      last = atomicInc(w.ctr, ng - 1) == ng - 1;
      if (last) {
        // Every group has merged: decode the ids, leave the slots at zero.
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint64_t m = __hip_atomic_exchange(w.slot + n, (uint64_t)0, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t row = ~(uint32_t)(m & 0xffffffffu);
          ids[n] = map.row_ids ? map.row_ids[row] : (int32_t)row;
        }
      }
    }
  }
}

template <int F, int NT, int LPR, bool XF32, bool BIG>
static hipError_t lm_launch_t(const DevInfo& dev, LmMap map, float* logits, int64_t ld,
                              const char* x, int64_t ldx_bytes, int C, char* ws,
                              int32_t* ids, hipStream_t s) {
  constexpr int G = (kWave / LPR) * Tune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  auto fn = lmhead_kernel<F, NT, LPR, XF32, BIG>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t n_groups = (map.V + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, kBlock);
  if (blocks > need) blocks = need;
  if (blocks > kLmMaxBlocks) blocks = kLmMaxBlocks;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &logits, &ld, (void*)&x, &ldx_bytes, &C, &ws, &ids};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
}

template <int F, int LPR, bool XF32>
static hipError_t lm_launch_nt(const DevInfo& dev, int nt, LmMap map, float* logits, int64_t ld,
                               const char* x, int64_t ldx_bytes, int C, char* ws, int32_t* ids,
                               hipStream_t s) {
#define Q8_LM(NTV, BIGV) \
  return lm_launch_t<F, NTV, LPR, XF32, BIGV>(dev, map, logits, ld, x, ldx_bytes, C, ws, ids, s)
  switch (nt) {
    case 1:
      if (map.V >= kBigRows) Q8_LM(1, true);
      Q8_LM(1, false);
    case 2: Q8_LM(2, false);
    case 3: Q8_LM(3, false);
    case 4: Q8_LM(4, false);
    case 5: Q8_LM(5, false);
    case 6: Q8_LM(6, false);
    case 7: Q8_LM(7, false);
    case 8: Q8_LM(8, false);
  }
#undef Q8_LM
  return hipErrorInvalidValue;
}

size_t lmhead_ws_bytes() { return kLmWsBytes; }

hipError_t launch_lmhead(const DevInfo& dev, const HMat& W, const int32_t* row_ids, const void* x,
                         bool x_f32, float* logits, int64_t ld_logits, int32_t* ids, char* ws,
                         int nt, hipStream_t s) {
  LmMap map;
  map.w = MatDesc{W.qs, W.d, W.ld_qs, W.ld_d};
  map.V = W.M;
  map.row_ids = row_ids;
  const int C = (int)chunks_per_row(W.fmt, W.K);
  const int64_t ldx_bytes = W.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  return dispatch_chunks(W.fmt, lanes_for(W.fmt, W.K), x_f32, [&](auto f, auto l, auto xf) {
    return lm_launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, ws, ids, s);
  });
}

}  // namespace q8
