// q8_gemv.hip -- dense Q8_0 GEMV and the fused gate+up pair (gfx950).
//
// One persistent launch per pass of up to 8 tokens. Workgroups stage x
// into LDS once, then their waves walk row groups with a grid stride, so
// every weight byte is fetched from HBM exactly once per pass and x is
// reused from LDS for all rows (memra wiki, feature list: Q8_0 decode
// matvecs with per-shape auto-dispatch; here the shape picks the lanes per
// row and the token count picks the rows per team).
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

// Rows [0, Ma) come from matrix A, rows [Ma, Mtot) from matrix B (the pair).
// Scalar fields and explicit selects: a struct-member select here was
// lowered to a private-memory array.
struct DenseMap {
  const int8_t* qa;
  const uint16_t* da;
  const int8_t* qb;
  const uint16_t* db;
  int64_t ldqa, ldda, ldqb, lddb;
  int64_t Ma, Mtot;
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    const bool second = i >= Ma;
    const int64_t k = second ? i - Ma : i;
    const int64_t ldq = second ? ldqb : ldqa;
    const int64_t ldd = second ? lddb : ldda;
    q = (second ? qb : qa) + k * ldq;
    d = (second ? db : da) + k * ldd;
    return i < Mtot;
  }
};

struct DenseEpi {
  char* ya;
  char* yb;
  int64_t Ma, Mtot;
  bool f16;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = base + i;
      if (idx >= NT * R) continue;
      const int n = idx / R, r = idx - (idx / R) * R;
      const int64_t row = rbase + r;
      if (row >= Mtot) continue;
      char* y;
      int64_t col, ld;
      if (row < Ma) { y = ya; col = row; ld = Ma; }
      else { y = yb; col = row - Ma; ld = Mtot - Ma; }
      if (f16) reinterpret_cast<_Float16*>(y)[n * ld + col] = (_Float16)v[i];
      else reinterpret_cast<float*>(y)[n * ld + col] = v[i];
    }
  }
};

template <int F, int NT, int LPR, bool XF32, int MODE>
__global__ __launch_bounds__(kBlock) void gemv_kernel(DenseMap map, DenseEpi epi, const char* x,
                                                      int64_t ldx_bytes, int C) {
  extern __shared__ uint4 lds_x[];
  using T = TuneM<NT, MODE>;
  constexpr int G = (kWave / LPR) * T::R;
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
    stage_fmt<F, NT, XF32>(rows, C, lds_x);
    __syncthreads();
  };
  run_rows<NT, LPR, T::R, T::D, 1, XF32, F>(map, epi, lds_x, C, n_groups,
                                            (int64_t)blockIdx.x * kWavesPerBlock + wave,
                                            (int64_t)gridDim.x * kWavesPerBlock, 0, stage);
}

// Chunks in flight per lane for run_once: all of them up to three, two up
// to seven, four from eight. Measured on MI355X at N = 1 (us, windows of
// 1 / 2 / up to 4 chunks): 5120 x 5120 (5 chunks per lane) 6.91 / 6.60 /
// 7.38; 8192 x 4096 (4) 7.77 / 7.77 / 8.08; 2048 x 768 (3) 3.33 / 3.36 /
// 3.01; 1024 x 16384 (16) 8.24 / 8.07 / 6.71. A runtime choice between
// windows (three copies of the loop in one kernel) cost up to 9% on small
// shapes, so the window follows the chunk count alone.
constexpr int once_depth(int cpl) { return cpl <= 3 ? cpl : cpl < 8 ? 2 : 4; }

// One token, at most one row group per wave, C = CPL * LPR: run_once. The
// workgroup size is chosen per launch (once_waves), up to 16 waves.
template <int F, int LPR, bool XF32, int CPL>
__global__ __launch_bounds__(kOnceMaxBlock) void gemv_once_kernel(DenseMap map, DenseEpi epi,
                                                                  const char* x, int C) {
  extern __shared__ uint4 lds_x[];
  constexpr int G = kWave / LPR;
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  auto stage = [=]() {
    const char* rows[1] = {x};
    stage_fmt<F, 1, XF32>(rows, C, lds_x);
    __syncthreads();
  };
  const int64_t g = (int64_t)blockIdx.x * waves + wave;
  run_once<1, LPR, 1, CPL, once_depth(CPL), 1, XF32, F>(
      map, epi, lds_x, lds_x + CPL * LPR * ChunkPlanes<F, XF32>::P, n_groups, g, 0, map.Mtot - 1,
      stage);
}


// ---------------------------------------------------------------- gate/up + SiLU
// The gate and up rows of output rho are virtual rows 2*rho and 2*rho + 1,
// so a team (an even number of rows) holds both sums of an output in one
// lane after the reduction and the MLP activation h = silu(g) * u is
// applied before anything is stored. Per-row arithmetic is the engine's, so
// g and u are bitwise those of q8_gemv_pair.
struct GluMap {
  const int8_t* qg;
  const uint16_t* dg;
  const int8_t* qu;
  const uint16_t* du;
  int64_t ldqg, lddg, ldqu, lddu;
  int64_t M2;  // 2 * M virtual rows
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    const int64_t rho = i >> 1;
    const bool up = (i & 1) != 0;
    const int64_t ldq = up ? ldqu : ldqg;
    const int64_t ldd = up ? lddu : lddg;
    q = (up ? qu : qg) + rho * ldq;
    d = (up ? du : dg) + rho * ldd;
    return i < M2;
  }
};

struct GluEpi {
  char* h;
  int64_t M;
  bool f16;
  template <int NT, int R, int CNT>
  __device__ __forceinline__ void emit(int64_t rbase, int base, bool owner, const float* v) {
    static_assert(R % 2 == 0 && CNT == 2, "gate/up pairs");
    if (!owner || base >= NT * R) return;
    const int n = base / R, r = base - (base / R) * R;
    const int64_t row = rbase + r;  // the gate row of the pair (even)
    if (row >= 2 * M) return;
    const float g = v[0], u = v[1];
    const float val = g / (1.0f + expf(-g)) * u;
    const int64_t o = (int64_t)n * M + (row >> 1);
    if (f16) reinterpret_cast<_Float16*>(h)[o] = (_Float16)val;
    else reinterpret_cast<float*>(h)[o] = val;
  }
};

template <int NT, bool BIG>
struct GluTune {
  static constexpr int R = Tune<NT, BIG>::R < 2 ? 2 : Tune<NT, BIG>::R;
};

template <int F, int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(kBlock) void glu_kernel(GluMap map, GluEpi epi, const char* x,
                                                     int64_t ldx_bytes, int C) {
  extern __shared__ uint4 lds_x[];
  constexpr int R = GluTune<NT, BIG>::R;
  constexpr int G = (kWave / LPR) * R;
  const int64_t n_groups = (map.M2 + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  auto stage = [=]() {
    const char* rows[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
    stage_fmt<F, NT, XF32>(rows, C, lds_x);
    __syncthreads();
  };
  run_rows<NT, LPR, R, 1, 2, XF32, F>(map, epi, lds_x, C, n_groups,
                                      (int64_t)blockIdx.x * kWavesPerBlock + wave,
                                      (int64_t)gridDim.x * kWavesPerBlock, 0, stage);
}

template <int F, int NT, int LPR, bool XF32, bool BIG>
static hipError_t glu_launch_t(const DevInfo& dev, GluMap map, GluEpi epi, const char* x,
                               int64_t ldx_bytes, int C, hipStream_t s) {
  constexpr int G = (kWave / LPR) * GluTune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  const int64_t n_groups = (map.M2 + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  auto fn = glu_kernel<F, NT, LPR, XF32, BIG>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, kBlock);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
}

template <int F, int LPR, bool XF32>
static hipError_t glu_launch_nt(const DevInfo& dev, int nt, GluMap map, GluEpi epi, const char* x,
                                int64_t ldx_bytes, int C, hipStream_t s) {
  switch (nt) {
    case 1:
      if (map.M2 >= kBigRows)
        return glu_launch_t<F, 1, LPR, XF32, true>(dev, map, epi, x, ldx_bytes, C, s);
      return glu_launch_t<F, 1, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 2: return glu_launch_t<F, 2, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 3: return glu_launch_t<F, 3, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 4: return glu_launch_t<F, 4, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 5: return glu_launch_t<F, 5, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 6: return glu_launch_t<F, 6, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 7: return glu_launch_t<F, 7, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
    case 8: return glu_launch_t<F, 8, LPR, XF32, false>(dev, map, epi, x, ldx_bytes, C, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_glu(const DevInfo& dev, const HMat& Gm, const HMat& Um, const void* x,
                      bool x_f32, void* h, bool h_f16, int nt, hipStream_t s) {
  GluMap map;
  map.qg = Gm.qs;
  map.dg = Gm.d;
  map.qu = Um.qs;
  map.du = Um.d;
  map.ldqg = Gm.ld_qs;
  map.lddg = Gm.ld_d;
  map.ldqu = Um.ld_qs;
  map.lddu = Um.ld_d;
  map.M2 = 2 * Gm.M;
  GluEpi epi;
  epi.h = (char*)h;
  epi.M = Gm.M;
  epi.f16 = h_f16;
  const int C = (int)chunks_per_row(Gm.fmt, Gm.K);
  const int64_t ldx_bytes = Gm.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  return dispatch_chunks(Gm.fmt, lanes_for(Gm.fmt, Gm.K), x_f32, [&](auto f, auto l, auto xf) {
    return glu_launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, epi, xp, ldx_bytes, C, s);
  });
}

template <int F, int NT, int LPR, bool XF32, int MODE>
static hipError_t launch_t(const DevInfo& dev, DenseMap map, DenseEpi epi, const char* x,
                           int64_t ldx_bytes, int C, hipStream_t s) {
  constexpr int G = (kWave / LPR) * TuneM<NT, MODE>::R;
  const size_t lds = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  auto fn = gemv_kernel<F, NT, LPR, XF32, MODE>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, kBlock);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
}

template <int F, int NT, int LPR, bool XF32>
static hipError_t launch_sz(const DevInfo& dev, DenseMap map, DenseEpi epi, const char* x,
                            int64_t ldx_bytes, int C, hipStream_t s) {
  if (NT == 1 && map.Mtot >= kBigRows)
    return launch_t<F, NT, LPR, XF32, 1>(dev, map, epi, x, ldx_bytes, C, s);
  // Small-matrix mode when the usual row groups cannot occupy the chip:
  // at most two groups per CU, or (for N >= 2, where teams carry 2-4 rows)
  // fewer groups than the chip's wave slots. Measured on MI355X: 5120 x
  // 5120 at N = 2, 4, 8 runs 5%, 8% and 11% faster, 2048 x 768 at N = 1
  // 8% faster; with ~20 groups per CU (5120 x 5120, N = 1) the deeper
  // window is 5% slower, so N = 1 keeps the usual mode there.
  constexpr int G0 = (kWave / LPR) * TuneM<NT, 0>::R;
  const int64_t groups = (map.Mtot + G0 - 1) / G0;
  if (groups <= 2 * (int64_t)dev.cus || (NT > 1 && groups < (int64_t)dev.cus * 32))
    return launch_t<F, NT, LPR, XF32, 2>(dev, map, epi, x, ldx_bytes, C, s);
  return launch_t<F, NT, LPR, XF32, 0>(dev, map, epi, x, ldx_bytes, C, s);
}

// Waves per workgroup for a one-group-per-wave launch of n_groups waves: 8,
// unless the launch gives the compute units at least 8 waves each and
// another resident size spreads them more evenly (the first in the order
// 10, 16, 5, 4 among the most even). Measured on MI355X at N = 1 (us,
// sweeps of 4, 5, 8, 10 and 16 waves): 5120 x 5120 10 waves 6.60 against 8
// waves 6.86 (640 workgroups, 2 or 3 per CU); with fewer waves per CU
// larger workgroups win, e.g. 1024 x 16384 8 waves 6.71 against 4 waves
// 7.43 (each workgroup stages all of x).
// LDS per workgroup: lds_fixed plus lds_per_wave for each wave.
static int once_waves(const DevInfo& dev, const void* fn, int64_t n_groups, size_t lds_fixed,
                      size_t lds_per_wave) {
  static const int kSizes[] = {8, 10, 16, 5, 4};
  const bool spread = n_groups >= 8 * (int64_t)dev.cus;
  int best = 0;
  double best_eff = 0.0;
  for (int w : kSizes) {
    const int64_t blocks = (n_groups + w - 1) / w;
    const int64_t per_cu = (blocks + dev.cus - 1) / dev.cus;
    const size_t lds = lds_fixed + (size_t)w * lds_per_wave;
    if (lds > dev.lds_per_block || per_cu > blocks_per_cu(fn, lds, w * kWave)) continue;
    const double eff = (double)n_groups / ((double)dev.cus * (double)per_cu * w);
    if (best == 0 || (spread && eff > best_eff + 1e-9)) {
      best = w;
      best_eff = eff;
    }
  }
  return best;
}

// The one-group-per-wave launch for N = 1 when the row groups fit in the
// resident waves and C is a whole number of lane steps with an instantiated
// count; hipErrorNotSupported when it does not apply (the caller then takes
// the persistent launch). Measured on MI355X, 5120 x 5120: 7.6 -> 6.4 us.
template <int F, int LPR, bool XF32, int CPL>
static hipError_t once_launch_t(const DevInfo& dev, DenseMap map, DenseEpi epi, const char* x,
                                int C, hipStream_t s) {
  constexpr int G = kWave / LPR;
  const size_t lds_x = (size_t)C * 16 * ChunkPlanes<F, XF32>::P;
  const size_t lds_wave = (size_t)G * row_scale_pieces(F, C) * 16;  // a wave's scale rows
  auto fn = gemv_once_kernel<F, LPR, XF32, CPL>;
  if (lds_x + kOnceMaxBlock / kWave * lds_wave > 64 * 1024) {
    const size_t most = std::min(lds_x + kOnceMaxBlock / kWave * lds_wave, dev.lds_per_block);
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)most);
    if (e != hipSuccess) return e;
  }
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int w = once_waves(dev, (const void*)fn, n_groups, lds_x, lds_wave);
  if (w == 0) return hipErrorNotSupported;
  const size_t lds = lds_x + (size_t)w * lds_wave;
  const int64_t blocks = (n_groups + w - 1) / w;
  void* args[] = {&map, &epi, (void*)&x, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(w * kWave), args, lds, s);
}

template <int F, int LPR, bool XF32>
static hipError_t once_launch(const DevInfo& dev, DenseMap map, DenseEpi epi, const char* x,
                              int C, hipStream_t s) {
  if (C % LPR != 0) return hipErrorNotSupported;
  switch (C / LPR) {
#define Q8_ONCE(N) \
  case N: return once_launch_t<F, LPR, XF32, N>(dev, map, epi, x, C, s);
    Q8_ONCE(1) Q8_ONCE(2) Q8_ONCE(3) Q8_ONCE(4) Q8_ONCE(5) Q8_ONCE(6) Q8_ONCE(7) Q8_ONCE(8)
    Q8_ONCE(10) Q8_ONCE(12) Q8_ONCE(14) Q8_ONCE(16)
#undef Q8_ONCE
  }
  return hipErrorNotSupported;
}

template <int F, int LPR, bool XF32>
static hipError_t launch_nt(const DevInfo& dev, int nt, DenseMap map, DenseEpi epi, const char* x,
                            int64_t ldx_bytes, int C, hipStream_t s) {
  switch (nt) {
    case 1:
      {
        const hipError_t e = once_launch<F, LPR, XF32>(dev, map, epi, x, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 1, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 2: return launch_sz<F, 2, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 3: return launch_sz<F, 3, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 4: return launch_sz<F, 4, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 5: return launch_sz<F, 5, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 6: return launch_sz<F, 6, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 7: return launch_sz<F, 7, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 8: return launch_sz<F, 8, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
  }
  return hipErrorInvalidValue;
}

int blocks_per_cu(const void* fn, size_t lds, int threads) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, size_t, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(fn, lds, threads);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n < 1) n = 1;
  cache[key] = n;
  return n;
}

int lanes_per_row(int64_t K) {
  const int64_t C = K / 16;
  if (C % 64 == 0) return 64;
  if (C % 32 == 0) return 32;
  if (C % 16 == 0) return 16;
  if (C >= 64) return 64;
  if (C >= 32) return 32;
  return 16;
}

int max_tokens_per_pass(const DevInfo& dev, int64_t K, bool x_f32) {
  const size_t per = x_lds_bytes(1, K, x_f32);
  if (per == 0) return kMaxNT;
  size_t n = dev.lds_per_block / per;
  if (n > (size_t)kMaxNT) n = kMaxNT;
  return (int)n;
}

hipError_t launch_gemv(const DevInfo& dev, const HMat& A, const HMat* B, const void* x,
                       bool x_f32, int64_t ldx, void* ya, void* yb, bool y_f16, int nt,
                       hipStream_t s) {
  DenseMap map;
  map.qa = A.qs;
  map.da = A.d;
  map.ldqa = A.ld_qs;
  map.ldda = A.ld_d;
  map.qb = B ? B->qs : A.qs;
  map.db = B ? B->d : A.d;
  map.ldqb = B ? B->ld_qs : A.ld_qs;
  map.lddb = B ? B->ld_d : A.ld_d;
  map.Ma = A.M;
  map.Mtot = A.M + (B ? B->M : 0);
  DenseEpi epi;
  epi.ya = (char*)ya;
  epi.yb = (char*)yb;
  epi.Ma = map.Ma;
  epi.Mtot = map.Mtot;
  epi.f16 = y_f16;
  const int C = (int)chunks_per_row(A.fmt, A.K);
  const int64_t ldx_bytes = ldx * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  return dispatch_chunks(A.fmt, lanes_for(A.fmt, A.K), x_f32, [&](auto f, auto l, auto xf) {
    return launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, epi, xp, ldx_bytes, C, s);
  });
}

}  // namespace q8
