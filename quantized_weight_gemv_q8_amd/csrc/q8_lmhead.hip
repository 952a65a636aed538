// q8_lmhead.hip -- LM-head Q8_0 GEMV fused with a greedy argmax (gfx950).
//
// The decode step ends with the vocabulary projection and a greedy pick;
// the pages keep the logits lean and move 4 bytes per token to the host
// (memra wiki, feature list: "CUDA-graph decode ... 4 bytes/token host
// traffic"), and greedy argmax is their correctness instrument (memra wiki,
// gate paragraph: run-gen prints its argmax gate before any number).
//
// Pass structure: one persistent GEMV launch whose workgroups each fold
// the rows they produced into one 64-bit key per token, written to a
// per-workgroup slot (no atomics, no pre-zeroed memory, deterministic),
// then a single-workgroup launch that takes the maximum key per token and
// decodes the row index. Key = (order-preserving bits of the fp32 logit,
// with -0 mapped to +0) << 32 | ~row, so the maximum key is the largest
// logit and, among equal logits, the lowest row.
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
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    q = w.qs + i * w.ld_qs;
    d = w.d + i * w.ld_d;
    return i < V;
  }
};

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
    my_base = base;
    my_owner = owner;
    if (!owner) return;
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

template <int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(kBlock) void lmhead_kernel(LmMap map, float* logits, int64_t ld,
                                                        const char* x, int64_t ldx_bytes, int C,
                                                        uint64_t* keys) {
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
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
    stage_x<NT, XF32>(rows, C, lds_x);
    __syncthreads();
  };
  run_rows<NT, LPR, R, T::D, 1, XF32>(map, epi, lds_x, C, n_groups,
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
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor(k, off, kWave);
      k = o > k ? o : k;
    }
    if (lane == 0) red[wave][n] = k;
  }
  __syncthreads();
  if (threadIdx.x < NT) {
    uint64_t k = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const uint64_t o = red[w][threadIdx.x];
      k = o > k ? o : k;
    }
    keys[(int64_t)blockIdx.x * NT + threadIdx.x] = k;
  }
}

// One workgroup: maximum key per token over the per-workgroup slots,
// decoded to the row index.
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void lmhead_final_kernel(const uint64_t* keys,
                                                                    int nblocks, int nt,
                                                                    int32_t* ids) {
  __shared__ uint64_t red[kFinalThreads / kWave][kMaxNT];
  uint64_t k[kMaxNT];
#pragma unroll
  for (int n = 0; n < kMaxNT; ++n) k[n] = 0;
  for (int b = threadIdx.x; b < nblocks; b += blockDim.x) {
#pragma unroll
    for (int n = 0; n < kMaxNT; ++n) {
      if (n < nt) {
        const uint64_t o = keys[(int64_t)b * nt + n];
        k[n] = o > k[n] ? o : k[n];
      }
    }
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int n = 0; n < kMaxNT; ++n) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor(k[n], off, kWave);
      k[n] = o > k[n] ? o : k[n];
    }
    if (lane == 0) red[wave][n] = k[n];
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    uint64_t m = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
      const uint64_t o = red[w][threadIdx.x];
      m = o > m ? o : m;
    }
    ids[threadIdx.x] = (int32_t)(~(uint32_t)(m & 0xffffffffu));
  }
}

int lmhead_blocks(const DevInfo& dev, int64_t V) {
  (void)dev;
  (void)V;
  return kLmMaxBlocks;
}

template <int NT, int LPR, bool XF32, bool BIG>
static hipError_t lm_launch_t(const DevInfo& dev, LmMap map, float* logits, int64_t ld,
                              const char* x, int64_t ldx_bytes, int C, uint64_t* keys,
                              int32_t* ids, hipStream_t s) {
  constexpr int G = (kWave / LPR) * Tune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * XPlanes<XF32>::P;
  auto fn = lmhead_kernel<NT, LPR, XF32, BIG>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t n_groups = (map.V + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds);
  if (blocks > need) blocks = need;
  if (blocks > kLmMaxBlocks) blocks = kLmMaxBlocks;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &logits, &ld, (void*)&x, &ldx_bytes, &C, &keys};
  hipError_t e = hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
  if (e != hipSuccess) return e;
  int nb = (int)blocks;
  int nt = NT;
  void* fargs[] = {&keys, &nb, &nt, &ids};
  return hipLaunchKernel((const void*)lmhead_final_kernel, dim3(1), dim3(kFinalThreads), fargs, 0,
                         s);
}

template <int LPR, bool XF32>
static hipError_t lm_launch_nt(const DevInfo& dev, int nt, LmMap map, float* logits, int64_t ld,
                               const char* x, int64_t ldx_bytes, int C, uint64_t* keys,
                               int32_t* ids, hipStream_t s) {
  switch (nt) {
    case 1:
      if (map.V >= kBigRows)
        return lm_launch_t<1, LPR, XF32, true>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
      return lm_launch_t<1, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 2: return lm_launch_t<2, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 3: return lm_launch_t<3, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 4: return lm_launch_t<4, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 5: return lm_launch_t<5, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 6: return lm_launch_t<6, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 7: return lm_launch_t<7, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
    case 8: return lm_launch_t<8, LPR, XF32, false>(dev, map, logits, ld, x, ldx_bytes, C, keys, ids, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lmhead(const DevInfo& dev, const HMat& W, const void* x, bool x_f32,
                         float* logits, int64_t ld_logits, int32_t* ids, uint64_t* keys, int nt,
                         hipStream_t s) {
  LmMap map;
  map.w = MatDesc{W.qs, W.d, W.ld_qs, W.ld_d};
  map.V = W.M;
  const int C = (int)(W.K / 16);
  const int64_t ldx_bytes = W.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int lpr = lanes_per_row(W.K);
  if (x_f32) {
    if (lpr == 64) return lm_launch_nt<64, true>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
    if (lpr == 32) return lm_launch_nt<32, true>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
    return lm_launch_nt<16, true>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
  }
  if (lpr == 64) return lm_launch_nt<64, false>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
  if (lpr == 32) return lm_launch_nt<32, false>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
  return lm_launch_nt<16, false>(dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, keys, ids, s);
}

}  // namespace q8
