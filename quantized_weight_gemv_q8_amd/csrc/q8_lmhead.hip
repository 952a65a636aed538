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
#include "q8_dense.h"
#include "q8_lmhead.h"

namespace q8 {

template <int F, int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(kBlock) void lmhead_kernel(LmMap map, float* logits, int64_t ld,
                                                        const char* x, int64_t ldx_bytes, int C,
                                                        char* ws, int32_t* ids) {
  extern __shared__ uint4 lds_x[];
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

  lm_merge<NT, R, CNT>(epi, map, ws, ids, kWavesPerBlock);
}

template <int F, int NT, int LPR, bool XF32, bool BIG>
static hipError_t lm_launch_t(const DevInfo& dev, LmMap map, float* logits, int64_t ld,
                              const char* x, int64_t ldx_bytes, int C, char* ws,
                              int32_t* ids, hipStream_t s) {
  constexpr int G = (kWave / LPR) * Tune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  auto fn = lmhead_kernel<F, NT, LPR, XF32, BIG>;
  if (hipError_t e = allow_dynamic_lds((const void*)fn, lds)) return e;
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

// Argmax over logits already in memory (the second launch of the two-launch
// head): each thread keeps the best key of a strided run of rows per token,
// and the workgroups merge as the fused kernel's do.
template <int NT>
__global__ __launch_bounds__(kBlock) void lm_argmax_kernel(const float* logits, int64_t ld,
                                                           int64_t V, const int32_t* row_ids,
                                                           char* ws, int32_t* ids) {
  uint64_t key[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) key[n] = 0;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x; v < V; v += stride) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint64_t k = argmax_key(logits[n * ld + v], v);
      key[n] = k > key[n] ? k : key[n];
    }
  }
  lm_merge_keys<NT>(key, row_ids, ws, ids, kWavesPerBlock);
}

// With logits requested at 1 or 2 tokens the head runs as the dense GEMV
// (the one-group kernel, which streams large vocabularies at ~90% of HBM
// peak) writing the logits, then lm_argmax_kernel over them: measured on
// MI355X, 151936 x 5120 N = 1, 114.3 us for the GEMV against 125.2 us for
// the fused kernel. The logits are bitwise those of the fused kernel (same
// per-row arithmetic), so are the ids. hipErrorNotSupported when the GEMV
// kernel does not apply.
static hipError_t lmhead_two_launch(const DevInfo& dev, const HMat& W, const int32_t* row_ids,
                                    const char* x, bool x_f32, int64_t ldx_bytes, int C,
                                    float* logits, int64_t ld, int32_t* ids, char* ws, int nt,
                                    hipStream_t s) {
  DenseMap map;
  map.qa = map.qb = W.qs;
  map.da = map.db = W.d;
  map.ldqa = map.ldqb = W.ld_qs;
  map.ldda = map.lddb = W.ld_d;
  map.Ma = map.Mtot = W.M;
  DenseEpi epi;
  epi.ya = epi.yb = (char*)logits;
  epi.Ma = epi.Mtot = W.M;
  epi.f16 = false;
  if (ld != W.M) return hipErrorNotSupported;
  hipError_t e = launch_gemv_once(nt, dev, map, epi, W.fmt, lanes_for(W.fmt, W.K), x_f32, x,
                                  ldx_bytes, C, s);
  if (e != hipSuccess) return e;
  int64_t blocks = (W.M + 4 * kBlock - 1) / (4 * kBlock);  // about four rows per thread
  if (blocks > 2 * (int64_t)dev.cus) blocks = 2 * (int64_t)dev.cus;
  int64_t V = W.M;
  void* args[] = {(void*)&logits, &ld, &V, (void*)&row_ids, &ws, &ids};
  const void* fn = nt == 1 ? (const void*)lm_argmax_kernel<1> : (const void*)lm_argmax_kernel<2>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlock), args, 0, s);
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
  if (logits && nt <= 2) {
    const hipError_t e = lmhead_two_launch(dev, W, row_ids, xp, x_f32, ldx_bytes, C, logits,
                                           ld_logits, ids, ws, nt, s);
    if (e != hipErrorNotSupported) return e;
  }
  return dispatch_chunks(W.fmt, lanes_for(W.fmt, W.K), x_f32, [&](auto f, auto l, auto xf) {
    return lm_launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, ws, ids, s);
  });
}

}  // namespace q8
