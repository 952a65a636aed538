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

#include "q8_dense.h"
#include "q8_engine.hpp"
#include "q8_internal.h"
#include "q8_once.hpp"

namespace q8 {

// One-group-per-wave launches by token count (instantiated in q8_once.hip).
hipError_t launch_gemv_once(int nt, const DevInfo& dev, const DenseMap& map, const DenseEpi& epi,
                            int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                            hipStream_t s, int slices) {
  switch (nt) {
#define Q8_ONCE_CASE(N) \
  case N:                                                                                     \
    return launch_once_nt<DenseKind, N>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s, slices);
    Q8_ONCE_CASE(1) Q8_ONCE_CASE(2) Q8_ONCE_CASE(3) Q8_ONCE_CASE(4)
    Q8_ONCE_CASE(5) Q8_ONCE_CASE(6) Q8_ONCE_CASE(7) Q8_ONCE_CASE(8)
#undef Q8_ONCE_CASE
  }
  return hipErrorNotSupported;
}

hipError_t launch_glu_once(int nt, const DevInfo& dev, const GluMap& map, const GluEpi& epi,
                           int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                           hipStream_t s, int slices) {
  switch (nt) {
#define Q8_ONCE_CASE(N) \
  case N:                                                                                     \
    return launch_once_nt<GluKind, N>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s, slices);
    Q8_ONCE_CASE(1) Q8_ONCE_CASE(2) Q8_ONCE_CASE(3) Q8_ONCE_CASE(4)
    Q8_ONCE_CASE(5) Q8_ONCE_CASE(6) Q8_ONCE_CASE(7) Q8_ONCE_CASE(8)
#undef Q8_ONCE_CASE
  }
  return hipErrorNotSupported;
}

template <int F, int NT, int LPR, bool XF32, int MODE>
__global__ __launch_bounds__(narrow_block<NT>()) __attribute__((
    amdgpu_waves_per_eu(narrow_waves_per_simd<F, NT, LPR, XF32>()))) void gemv_kernel(DenseMap map, DenseEpi epi, const char* x,
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
  constexpr int WPB = narrow_block<NT>() / kWave;
  run_rows<NT, LPR, T::R, T::D, 1, XF32, F>(map, epi, lds_x, C, n_groups,
                                            (int64_t)blockIdx.x * WPB + wave,
                                            (int64_t)gridDim.x * WPB, 0, stage);
}

// ---------------------------------------------------------------- 9..16 tokens
// Passes of 9 to 16 tokens (the K+1 verify at K = 8 and wider batched
// decode) run one persistent kernel per kind whose token count nt is a
// runtime value: tokens n >= nt are neither staged, computed nor stored, so
// every weight byte is read once for all of them instead of once per pass
// of 8. Four rows per team (so each LDS read of x serves four rows), two
// for the SiLU pair's 16-lane teams (whose reduction must leave one gate/up
// pair per lane). Per (row, token) the arithmetic is that of every other
// dense kernel, so the results stay bitwise N-invariant.
template <int LPR, bool GLU>
constexpr int wide_rows() { return GLU && LPR == 16 ? 2 : 4; }
// One workgroup per CU (a 16-token image of a 5120-wide x takes the whole
// LDS), so the workgroup holds as many waves as the registers allow. Q8_0
// weights, fp16 activations and 64-lane rows: two chunks in flight per
// wave (D = 2, 140 registers a lane) and 12 waves; measured on MI355X for
// the 2 x 17408 x 5120 pair, 16 waves with one chunk in flight take 81.6
// (N = 9) and 114.4 us (N = 16), 12 waves with two 70.2 and 96.7 us. Other
// formats and row widths (wider chunk or reduction state): one chunk in
// flight and 8 waves.
template <int F, int LPR, bool XF32>
constexpr bool wide_deep() { return F == kFmtQ8 && !XF32 && LPR == 64; }
template <int F, int LPR, bool XF32>
constexpr int wide_depth() { return wide_deep<F, LPR, XF32>() ? 2 : 1; }
template <int F, int LPR, bool XF32>
constexpr int wide_block() { return wide_deep<F, LPR, XF32>() ? 768 : 512; }

template <int F, int LPR, bool XF32, int MINC, int R, class Map, class Epi>
__device__ __forceinline__ void wide_body(const Map& map, Epi& epi, int64_t rows, const char* x,
                                          int64_t ldx_bytes, int C, int nt) {
  extern __shared__ uint4 lds_x[];
  constexpr int NT = kMaxNTWide;
  constexpr int G = (kWave / LPR) * R;
  const int64_t n_groups = (rows + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  auto stage = [=]() {
    const char* xr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) xr[n] = x + (n < nt ? n : 0) * ldx_bytes;
    stage_fmt<F, NT, XF32>(xr, C, lds_x, nt);
    __syncthreads();
  };
  const int wpb = (int)(blockDim.x / kWave);
  run_rows<NT, LPR, R, wide_depth<F, LPR, XF32>(), MINC, XF32, F>(map, epi, lds_x, C, n_groups,
                                              (int64_t)blockIdx.x * wpb + wave,
                                              (int64_t)gridDim.x * wpb, 0, stage, nt);
}

template <int F, int LPR, bool XF32>
__global__ __launch_bounds__((wide_block<F, LPR, XF32>())) void gemv_wide_kernel(DenseMap map, DenseEpi epi,
                                                           const char* x, int64_t ldx_bytes, int C,
                                                           int nt) {
  wide_body<F, LPR, XF32, 1, wide_rows<LPR, false>()>(map, epi, map.Mtot, x, ldx_bytes, C, nt);
}

template <int F, int LPR, bool XF32>
__global__ __launch_bounds__((wide_block<F, LPR, XF32>())) void glu_wide_kernel(GluMap map, GluEpi epi, const char* x,
                                                          int64_t ldx_bytes, int C, int nt) {
  wide_body<F, LPR, XF32, 2, wide_rows<LPR, true>()>(map, epi, map.M2, x, ldx_bytes, C, nt);
}

// Persistent launch of a wide kernel over `rows` virtual rows (nt tokens
// staged: nt * C * 16 * P bytes of LDS).
template <int F, int LPR, bool XF32, class Map, class Epi>
static hipError_t wide_launch(const DevInfo& dev, const void* fn, int G, Map map, Epi epi,
                              int64_t rows, const char* x, int64_t ldx_bytes, int C, int nt,
                              hipStream_t s) {
  const size_t lds = (size_t)nt * C * 16 * ChunkPlanes<F, XF32>::P;
  if (nt <= kMaxNT || nt > kMaxNTWide || lds > dev.lds_per_block) return hipErrorInvalidValue;
  if (hipError_t e = allow_dynamic_lds(fn, lds)) return e;
  // Waves per workgroup: as many as the row groups need for one workgroup
  // per CU, up to the kernel's maximum (a small matrix then still spreads
  // over every CU instead of filling a few CUs with 16 waves each).
  constexpr int WMAX = wide_block<F, LPR, XF32>() / kWave;
  const int64_t groups = (rows + G - 1) / G;
  int64_t w = (groups + dev.cus - 1) / dev.cus;
  if (w > WMAX) w = WMAX;
  if (w < 1) w = 1;
  const int threads = (int)w * kWave;
  const int64_t need = (groups + w - 1) / w;
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu(fn, lds, threads);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  epi.nt = nt;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C, &nt};
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), args, lds, s);
}

// ---------------------------------------------------------------- gate/up + SiLU
template <int NT, bool BIG>
struct GluTune {
  static constexpr int R = Tune<NT, BIG>::R < 2 ? 2 : Tune<NT, BIG>::R;
};

template <int F, int NT, int LPR, bool XF32, bool BIG>
__global__ __launch_bounds__(narrow_block<NT>()) __attribute__((
    amdgpu_waves_per_eu(narrow_waves_per_simd<F, NT, LPR, XF32>()))) void glu_kernel(GluMap map, GluEpi epi, const char* x,
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
                                      (int64_t)blockIdx.x * (narrow_block<NT>() / kWave) + wave,
                                      (int64_t)gridDim.x * (narrow_block<NT>() / kWave), 0, stage);
}

template <int F, int NT, int LPR, bool XF32, bool BIG>
static hipError_t glu_launch_t(const DevInfo& dev, GluMap map, GluEpi epi, const char* x,
                               int64_t ldx_bytes, int C, hipStream_t s) {
  constexpr int G = (kWave / LPR) * GluTune<NT, BIG>::R;
  const size_t lds = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  const int64_t n_groups = (map.M2 + G - 1) / G;
  constexpr int NB = narrow_block<NT>();
  const int64_t need = (n_groups + NB / kWave - 1) / (NB / kWave);
  auto fn = glu_kernel<F, NT, LPR, XF32, BIG>;
  if (hipError_t e = allow_dynamic_lds((const void*)fn, lds)) return e;
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, NB);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(NB), args, lds, s);
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
                      bool x_f32, void* h, bool h_f16, int nt, hipStream_t s, const HMat* extra,
                      float* xdot, int slices) {
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
  if (extra) {
    map.qx = extra->qs;
    map.dx = extra->d;
    map.M = Gm.M;
    map.M2 += 2;
  }
  GluEpi epi;
  epi.h = (char*)h;
  epi.M = Gm.M;
  epi.f16 = h_f16;
  epi.xdot = extra ? xdot : nullptr;
  const int C = (int)chunks_per_row(Gm.fmt, Gm.K);
  const int64_t ldx_bytes = Gm.K * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  if (slices > 1) {
    if (nt > kMaxNT) return hipErrorInvalidValue;
    const hipError_t e = launch_glu_once(nt, dev, map, epi, Gm.fmt, lanes_for(Gm.fmt, Gm.K),
                                         x_f32, xp, ldx_bytes, C, s, slices);
    if (e != hipErrorNotSupported) return e;
    for (int k = 0; k < slices; ++k) {
      const int n0 = k * nt;
      const hipError_t ek = launch_glu(dev, Gm, Um, xp + (int64_t)n0 * ldx_bytes, x_f32,
                                       (char*)h + (int64_t)n0 * Gm.M * (h_f16 ? 2 : 4), h_f16, nt,
                                       s, extra, xdot ? xdot + n0 : nullptr);
      if (ek != hipSuccess) return ek;
    }
    return hipSuccess;
  }
  if (nt > kMaxNT) {
    if (!wide_pass_applies(dev, Gm.fmt, Gm.K, x_f32, map.M2)) return hipErrorInvalidValue;
    return wide_launch<kFmtQ8, 64, false>(dev, (const void*)glu_wide_kernel<kFmtQ8, 64, false>,
                                          wide_rows<64, true>(), map, epi, map.M2, xp, ldx_bytes,
                                          C, nt, s);
  }
  {
    const hipError_t e = launch_glu_once(nt, dev, map, epi, Gm.fmt, lanes_for(Gm.fmt, Gm.K), x_f32,
                                         xp, ldx_bytes, C, s);
    if (e != hipErrorNotSupported) return e;
  }
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
  constexpr int NB = narrow_block<NT>();
  const int64_t need = (n_groups + NB / kWave - 1) / (NB / kWave);
  auto fn = gemv_kernel<F, NT, LPR, XF32, MODE>;
  if (hipError_t e = allow_dynamic_lds((const void*)fn, lds)) return e;
  int64_t blocks = (int64_t)dev.cus * blocks_per_cu((const void*)fn, lds, NB);
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(NB), args, lds, s);
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
  // window is 5% slower, so N = 1 keeps the usual mode there. Q4_0 passes
  // of 6 or more tokens over at least 8 groups per CU keep the usual mode
  // too (17408 x 5120, 8.5 groups per CU, at N = 6 and 8: 3% and 5%
  // faster; at N = 4 it is 11% slower).
  constexpr int G0 = (kWave / LPR) * TuneM<NT, 0>::R;
  const int64_t groups = (map.Mtot + G0 - 1) / G0;
  const bool q4_wide = F == kFmtQ4 && NT >= 6 && groups >= 8 * (int64_t)dev.cus;
  if (groups <= 2 * (int64_t)dev.cus || (NT > 1 && !q4_wide && groups < (int64_t)dev.cus * 32))
    return launch_t<F, NT, LPR, XF32, 2>(dev, map, epi, x, ldx_bytes, C, s);
  return launch_t<F, NT, LPR, XF32, 0>(dev, map, epi, x, ldx_bytes, C, s);
}

template <int F, int LPR, bool XF32>
static hipError_t launch_nt(const DevInfo& dev, int nt, DenseMap map, DenseEpi epi, const char* x,
                            int64_t ldx_bytes, int C, hipStream_t s) {
  switch (nt) {
    case 1:
      {
        const hipError_t e = launch_gemv_once(1, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 1, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 2:
      {
        const hipError_t e = launch_gemv_once(2, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 2, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 3:
      {
        const hipError_t e = launch_gemv_once(3, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 3, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 4:
      {
        const hipError_t e = launch_gemv_once(4, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 4, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 5:
      {
        const hipError_t e = launch_gemv_once(5, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 5, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 6:
      {
        const hipError_t e = launch_gemv_once(6, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 6, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 7:
      {
        const hipError_t e = launch_gemv_once(7, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 7, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 8:
      {
        const hipError_t e = launch_gemv_once(8, dev, map, epi, F, LPR, XF32, x, ldx_bytes, C, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch_sz<F, 8, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
  }
  return hipErrorInvalidValue;
}

hipError_t allow_dynamic_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int device = 0;
  if (hipError_t e = hipGetDevice(&device)) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> raised;  // per device and kernel
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(device, fn);
  auto it = raised.find(key);
  if (it != raised.end() && it->second >= bytes) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) raised[key] = bytes;
  return e;
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

int max_tokens_per_pass_wide(const DevInfo& dev, int64_t K, bool x_f32) {
  const size_t per = x_lds_bytes(1, K, x_f32);
  if (per == 0) return kMaxNTWide;
  size_t n = dev.lds_per_block / per;
  if (n > (size_t)kMaxNTWide) n = kMaxNTWide;
  return (int)n;
}

// Passes of 9..16 tokens run the wide kernel for Q8_0 weights, fp16
// activations and 64-lane rows, and only when the matrix has row groups for
// a full workgroup on every CU (groups of four rows, twelve waves): below
// that, the one-row-group-per-wave kernels of two passes of at most 8 are
// faster (measured on MI355X at 5120 x 5120: N = 9 and 16 in 21.4 and
// 27.6 us wide, against 17.4 and 23.7 us as two passes; the 2 x 17408 x
// 5120 pair, 34 row groups per CU, takes 70.2 and 96.7 us wide against 85
// and 114 us as two passes).
bool wide_pass_applies(const DevInfo& dev, int fmt, int64_t K, bool x_f32, int64_t rows) {
  if (fmt != kFmtQ8 || x_f32 || lanes_for(fmt, K) != 64) return false;
  const int64_t groups = (rows + 3) / 4;
  return groups >= (int64_t)(wide_block<kFmtQ8, 64, false>() / kWave) * dev.cus;
}

hipError_t launch_gemv(const DevInfo& dev, const HMat& A, const HMat* B, const void* x,
                       bool x_f32, int64_t ldx, void* ya, void* yb, bool y_f16, int nt,
                       hipStream_t s, const float* gate, int slices) {
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
  epi.gate = gate;
  const int C = (int)chunks_per_row(A.fmt, A.K);
  const int64_t ldx_bytes = ldx * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  if (slices > 1) {
    if (nt > kMaxNT) return hipErrorInvalidValue;
    const hipError_t e = launch_gemv_once(nt, dev, map, epi, A.fmt, lanes_for(A.fmt, A.K), x_f32,
                                          xp, ldx_bytes, C, s, slices);
    if (e != hipErrorNotSupported) return e;
    const int64_t ys = y_f16 && gate == nullptr ? 2 : 4;
    for (int k = 0; k < slices; ++k) {
      const int n0 = k * nt;
      const hipError_t ek = launch_gemv(
          dev, A, B, xp + (int64_t)n0 * ldx_bytes, x_f32, ldx, (char*)ya + n0 * A.M * ys,
          B ? (char*)yb + n0 * B->M * ys : nullptr, y_f16, nt, s, gate ? gate + n0 : nullptr);
      if (ek != hipSuccess) return ek;
    }
    return hipSuccess;
  }
  if (nt > kMaxNT) {
    if (!wide_pass_applies(dev, A.fmt, A.K, x_f32, map.Mtot)) return hipErrorInvalidValue;
    return wide_launch<kFmtQ8, 64, false>(dev, (const void*)gemv_wide_kernel<kFmtQ8, 64, false>,
                                          wide_rows<64, false>(), map, epi, map.Mtot, xp,
                                          ldx_bytes, C, nt, s);
  }
  return dispatch_chunks(A.fmt, lanes_for(A.fmt, A.K), x_f32, [&](auto f, auto l, auto xf) {
    return launch_nt<decltype(f)::value, decltype(l)::value, decltype(xf)::value>(
        dev, nt, map, epi, xp, ldx_bytes, C, s);
  });
}

}  // namespace q8
