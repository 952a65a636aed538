// q8_lmhead.hip -- LM-head Q8_0 GEMV fused with a greedy argmax (gfx950).
//
// The decode step ends with the vocabulary projection and a greedy pick;
// the pages keep the logits on the device and move only 4 bytes per token
// to the host (memra wiki, feature list, the graph-decode item), and greedy
// argmax is their correctness instrument (memra wiki, gate paragraph: the
// generation runner reports its argmax gate before any timing).
//
// Pass structure (passes of 3 to 8 tokens, one-token passes over small
// vocabularies, or where the one-group GEMV does not apply; the rest take
// the two-launch head below): one persistent GEMV launch. Each workgroup folds the
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
// and the workgroups merge as the fused kernel's do. With clear set the
// logits are the workspace's scratch rows and each is set back to zero
// once read.
constexpr int kLmArgU = 4;

template <int NT>
__global__ __launch_bounds__(kBlock) void lm_argmax_kernel(float* logits, int64_t ld, int64_t V,
                                                           const int32_t* row_ids, char* ws,
                                                           int32_t* ids, bool clear) {
  // kLmArgU rows per thread per step, all loaded before the first compare
  // (one memory round trip per step); the maximum does not depend on the
  // order, so neither do the ids.
  uint64_t key[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) key[n] = 0;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t v0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; v0 < V; v0 += kLmArgU * stride) {
    float val[kLmArgU][NT];
#pragma unroll
    for (int u = 0; u < kLmArgU; ++u) {
      const int64_t v = v0 + u * stride;
      const int64_t vc = v < V ? v : v0;
#pragma unroll
      for (int n = 0; n < NT; ++n) val[u][n] = logits[n * ld + vc];
    }
#pragma unroll
    for (int u = 0; u < kLmArgU; ++u) {
      const int64_t v = v0 + u * stride;
      if (v >= V) continue;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint64_t k = argmax_key(val[u][n], v);
        key[n] = k > key[n] ? k : key[n];
        if (clear) logits[n * ld + v] = 0.0f;
      }
    }
  }
  lm_merge_keys<NT>(key, row_ids, ws, ids, kWavesPerBlock);
}

// The two-launch head (two_launch_pays): the dense GEMV (the one-group
// kernel, which streams large vocabularies at ~90% of HBM peak) writes the
// logits -- the caller's, or with none requested the workspace's scratch
// rows -- then lm_argmax_kernel takes the argmax over them. Measured on MI355X, 151936 x 5120 N = 1:
// GEMV 115.4 us + argmax 5.1 us against 125 us for the fused kernel.
// Merging per-workgroup keys with atomics at the end of the one-group
// kernel instead was slower (127 us for the GEMV alone): each workgroup
// stays resident until its agent-scope atomic completes. The logits are
// bitwise those of the fused kernel (same per-row arithmetic), so are the
// ids. hipErrorNotSupported when the GEMV kernel does not apply.
static hipError_t lmhead_two_launch(const DevInfo& dev, const HMat& W, const int32_t* row_ids,
                                    const char* x, bool x_f32, int64_t ldx_bytes, int C,
                                    float* logits, int64_t ld, bool clear, int32_t* ids, char* ws,
                                    int nt, hipStream_t s) {
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
  int64_t blocks = (W.M + kLmArgU * kBlock - 1) / (kLmArgU * kBlock);  // one step per thread
  if (blocks > 2 * (int64_t)dev.cus) blocks = 2 * (int64_t)dev.cus;
  int64_t V = W.M;
  void* args[] = {(void*)&logits, &ld, &V, (void*)&row_ids, &ws, &ids, &clear};
  const void* fn = nt == 1 ? (const void*)lm_argmax_kernel<1> : (const void*)lm_argmax_kernel<2>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlock), args, 0, s);
}

// Whether the two-launch head is the faster at this shape. Its one-group
// GEMV streams at ~90% of HBM peak against the fused kernel's ~85%, and
// the second launch costs a few microseconds, so one token needs enough
// weight bytes; two tokens always gain. Measured on MI355X (us, fused ->
// two launches), ids only: 16000 x 4096 15.8 -> 17.5, 48000 x 4096 36.9 ->
// 37.7, 65536 x 4096 50.2 -> 47.1, 151936 x 5120 125.1 -> 120.0; with
// logits: 32000 x 4096 26.3 -> 26.8, 48000 x 4096 37.9 -> 36.9; two
// tokens: 16000 x 4096 23.9 -> 20.7, 151936 x 4096 121.4 -> 110.4.
static bool two_launch_pays(const HMat& W, int nt, bool logits) {
  if (nt > 2) return false;
  if (nt == 2) return true;
  const double bytes = (double)W.M * (double)W.K * (W.fmt == kFmtQ4 ? 18.0 : 34.0) / 32.0;
  return bytes >= (logits ? 150e6 : 280e6);
}

int lmhead_max_tokens_per_pass(const DevInfo& dev, int64_t K, bool x_f32) {
  const size_t per = x_lds_bytes(1, K, x_f32);
  if (dev.lds_per_block <= kLmStaticLds) return 0;
  size_t n = (dev.lds_per_block - kLmStaticLds) / per;
  if (n > (size_t)kMaxNT) n = kMaxNT;
  return (int)n;
}

// Slots and counters, then scratch logits for two tokens (256-byte aligned).
size_t lmhead_ws_bytes(int64_t V) {
  const size_t scratch = ((size_t)(V > 0 ? V : 0) * 2 * sizeof(float) + 255) / 256 * 256;
  return kLmWsBytes + scratch;
}

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
  if (two_launch_pays(W, nt, logits != nullptr)) {
    float* scratch = (float*)(ws + kLmWsBytes);
    const hipError_t e = lmhead_two_launch(dev, W, row_ids, xp, x_f32, ldx_bytes, C,
                                           logits ? logits : scratch, logits ? ld_logits : W.M,
                                           !logits, ids, ws, nt, s);
    if (e != hipErrorNotSupported) return e;
  }
  return dispatch_chunks(W.fmt, lanes_for(W.fmt, W.K), x_f32, [&](auto f, auto l, auto xf) {
    return lm_launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, logits, ld_logits, xp, ldx_bytes, C, ws, ids, s);
  });
}

}  // namespace q8
