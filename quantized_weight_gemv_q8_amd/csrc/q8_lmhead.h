// q8_lmhead.h -- the LM head's row map, workspace, per-lane running argmax
// and end-of-workgroup merge.
#pragma once
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

constexpr int kLmMaxBlocks = 4096;
// Static LDS of the fused head (lm_merge_keys' per-wave keys): the x image
// of a pass gets what is left of the workgroup's LDS.
constexpr size_t kLmStaticLds = sizeof(uint64_t) * (kOnceMaxBlock / kWave) * kMaxNT;

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

// End of a workgroup: merge each token's best key of the workgroup into
// the workspace slots, and let the last workgroup decode the ids (see the
// top of q8_lmhead.hip). key[n] is this lane's best key for token n (0 for
// none). Every thread of the workgroup calls it; waves <=
// kOnceMaxBlock / kWave.
template <int NT>
__device__ __forceinline__ void lm_merge_keys(const uint64_t* key, const int32_t* row_ids,
                                              char* ws, int32_t* ids, int waves) {
  __shared__ uint64_t red[kOnceMaxBlock / kWave][kMaxNT];
  static_assert(sizeof(red) == kLmStaticLds, "the pass size reserves exactly this");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint64_t k = wave_max_u64(key[n]);
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
      for (int wv = 0; wv < waves; ++wv) {
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
          ids[n] = row_ids ? row_ids[row] : (int32_t)row;
        }
      }
    }
  }
}

// The same from a workgroup's LmEpi running bests.
template <int NT, int R, int CNT>
__device__ __forceinline__ void lm_merge(const LmEpi<CNT>& epi, const LmMap& map, char* ws,
                                         int32_t* ids, int waves) {
  uint64_t key[NT];
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
    key[n] = k;
  }
  lm_merge_keys<NT>(key, map.row_ids, ws, ids, waves);
}

}  // namespace q8
