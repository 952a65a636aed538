// q8_once.hpp -- the dense GEMV with one row group per wave (run_once) for
// passes of 1 to 8 tokens: kernels, their launch shape and the launcher.
// q8_once.hip instantiates it for one kind and token count per build of
// that file (separate translation units so the build compiles them in
// parallel).
#pragma once
#include <algorithm>
#include <type_traits>

#include "q8_dense.h"
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

// Chunks in flight per lane for run_once: all of them up to three, two up
// to seven, four from eight. Measured on MI355X at N = 1 (us, windows of
// 1 / 2 / up to 4 chunks): 5120 x 5120 (5 chunks per lane) 6.91 / 6.60 /
// 7.38; 8192 x 4096 (4) 7.77 / 7.77 / 8.08; 2048 x 768 (3) 3.33 / 3.36 /
// 3.01; 1024 x 16384 (16) 8.24 / 8.07 / 6.71. A runtime choice between
// windows (three copies of the loop in one kernel) cost up to 9% on small
// shapes, so the window follows the chunk count alone.
constexpr int once_depth(int cpl) { return cpl <= 3 ? cpl : cpl < 8 ? 2 : 4; }

// Fewest tokens per pass of a one-group kernel that runs several passes
// per launch (blockIdx.y selects the pass); smaller passes take one launch
// each.
constexpr int kMinSliceNT = 4;

// Rows per team: one up to 4 tokens; two from 5, which halves the groups
// (so that 5120 rows fit in the waves the larger x image leaves resident)
// and shares each LDS read of x between two rows.
constexpr int once_rows(int nt) { return nt <= 4 ? 1 : 2; }

// The two kinds of one-group kernels: the dense GEMV (and pair) and the
// gate/up + SiLU pair, whose teams hold a gate row and its up row (R = 2,
// both sums reduced into one lane: MINC = 2).
struct DenseKind {
  using Map = DenseMap;
  using Epi = DenseEpi;
  static constexpr int rows_per_team(int nt) { return once_rows(nt); }
  static constexpr int kMinc = 1;
  __host__ __device__ static int64_t rows(const Map& m) { return m.Mtot; }
};
struct GluKind {
  using Map = GluMap;
  using Epi = GluEpi;
  static constexpr int rows_per_team(int) { return 2; }
  static constexpr int kMinc = 2;
  __host__ __device__ static int64_t rows(const Map& m) { return m.M2; }
};

// NT tokens, at most one row group per wave, C = CPL * LPR: run_once. The
// workgroup size is chosen per launch (once_waves), up to 16 waves. XB = 0
// stages x after the weight loads of the window are issued (LateStage);
// XB >= 1 loads it first, XB pieces per thread and token (EarlyStage).
template <class K, int F, int NT, int LPR, bool XF32, int CPL, int XB = 0,
          int D = once_depth(CPL), int RT = K::rows_per_team(NT), bool SYNC = false>
__device__ __forceinline__ void once_body(const typename K::Map& map, typename K::Epi& epi,
                                          const char* x, int64_t ldx_bytes, int C) {
  extern __shared__ uint4 lds_x[];
  constexpr int R = RT;
  constexpr int G = kWave / LPR * R;
  constexpr int P = ChunkPlanes<F, XF32>::P;
  const int64_t rows = K::rows(map);
  const int64_t n_groups = (rows + G - 1) / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  const int64_t g = (int64_t)blockIdx.x * waves + wave;
  uint4* const lds_s = lds_x + NT * CPL * LPR * P;
  // Pass blockIdx.y of a launch of several passes, which only kernels of
  // kMinSliceNT or more tokens take (the check alone made the one-token
  // kernel 1.5-2% slower on 5120 x 5120).
  if constexpr (NT >= kMinSliceNT) {
    if (blockIdx.y != 0) {
      x += (int64_t)blockIdx.y * NT * ldx_bytes;
      epi.shift((int)blockIdx.y * NT);
    }
  }
  if constexpr (XB > 0) {
    EarlyStage<NT, P, XB, SYNC> stage{x, ldx_bytes, C, NT, lds_x};
    run_once<NT, LPR, R, CPL, D, K::kMinc, XF32, F>(map, epi, lds_x, lds_s, n_groups, g, 0,
                                                    rows - 1, stage);
  } else {
    auto stage = late_stage([=]() {
      const char* xr[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) xr[n] = x + n * ldx_bytes;
      stage_fmt<F, NT, XF32>(xr, C, lds_x);
      __syncthreads();
    });
    run_once<NT, LPR, R, CPL, D, K::kMinc, XF32, F>(map, epi, lds_x, lds_s, n_groups, g, 0,
                                                    rows - 1, stage);
  }
}

template <int F, int NT, int LPR, bool XF32, int CPL, int XB = 0>
__global__ __launch_bounds__(kOnceMaxBlock) void gemv_once_kernel(DenseMap map, DenseEpi epi,
                                                                  const char* x,
                                                                  int64_t ldx_bytes, int C) {
  once_body<DenseKind, F, NT, LPR, XF32, CPL, XB>(map, epi, x, ldx_bytes, C);
}

template <int F, int NT, int LPR, bool XF32, int CPL, int XB = 0>
__global__ __launch_bounds__(kOnceMaxBlock) void glu_once_kernel(GluMap map, GluEpi epi,
                                                                 const char* x, int64_t ldx_bytes,
                                                                 int C) {
  once_body<GluKind, F, NT, LPR, XF32, CPL, XB>(map, epi, x, ldx_bytes, C);
}

template <class K, int F, int NT, int LPR, bool XF32, int CPL, int XB = 0>
constexpr const void* once_fn() {
  if constexpr (std::is_same_v<K, GluKind>)
    return (const void*)glu_once_kernel<F, NT, LPR, XF32, CPL, XB>;
  else
    return (const void*)gemv_once_kernel<F, NT, LPR, XF32, CPL, XB>;
}

// Two-token passes load x ahead of the weights (EarlyStage, one piece per
// thread and token) when a workgroup has a thread for every piece of a
// token's image. Measured on MI355X (same-process A/B, graph replay):
// 5120 x 5120 N = 2 7.48 -> 7.01 us; at N = 1 neither order is faster
// (6.42 against 6.45 us: there the barrier waits on the memory queue of the
// compute unit either way), so one-token passes keep the late staging.
constexpr bool once_early(int nt) { return nt == 2; }

// Waves per workgroup for a one-group-per-wave launch of n_groups waves: 8,
// unless the launch gives the compute units at least 8 waves each and
// another resident size spreads them more evenly (the first in the order
// 10, 16, 5, 4 among the most even), or gives them fewer (below).
// Measured on MI355X at N = 1 (us, sweeps of 4, 5, 8, 10 and 16 waves):
// 5120 x 5120 10 waves 6.60 against 8 waves 6.86 (640 workgroups, 2 or 3
// per CU); with fewer waves per CU larger workgroups win, e.g. 1024 x
// 16384 8 waves 6.71 against 4 waves 7.43 (each workgroup stages all of x).
// LDS per workgroup: lds_fixed plus lds_per_wave for each wave. With
// stream set, a launch whose groups do not all fit in the resident waves
// still takes this kernel with 8-wave workgroups, the hardware starting
// workgroups as others finish (0 otherwise: the caller takes the
// persistent launch). Measured on MI355X, one-group against persistent:
// 34816 x 5120 N = 1 30.3 -> 28.7 us, N = 2 36.5 -> 32.1; 102400 x 5120
// N = 1 87.5 -> 77.9; but N = 4 38.8 -> 43.0 and N = 8 57.2 -> 73.8 (each
// workgroup stages x again), so only passes of 1 or 2 tokens stream.
static int once_waves(const DevInfo& dev, const void* fn, int64_t n_groups, size_t lds_fixed,
                      size_t lds_per_wave, bool stream) {
  static const int kSizes[] = {8, 10, 16, 5, 4};
  const bool spread = n_groups >= 8 * (int64_t)dev.cus;
  // Fewer than 8 groups per CU: workgroups of ceil(groups / CUs) waves but
  // at least 4, so that every CU gets one where the groups allow (smaller
  // workgroups each stage x again). Measured on MI355X against 8-wave
  // workgroups (same-process A/B): 2048 x 768 N = 1 / 2 / 8 2.90 / 3.20 /
  // 6.21 -> 2.78 / 2.99 / 4.87 us, 1024 x 1024 N = 2 / 8 2.87 / 4.12 ->
  // 2.69 / 3.69, a 128 x 2048 router at 8-64 tokens 10% faster, the shared
  // expert 3%; with 1- to 3-wave workgroups the router lost up to 12%.
  if (!spread) {
    int64_t w = (n_groups + dev.cus - 1) / dev.cus;
    w = w < 4 ? 4 : w > 8 ? 8 : w;
    const size_t lds = lds_fixed + (size_t)w * lds_per_wave;
    const int64_t blocks = (n_groups + w - 1) / w;
    if (lds <= dev.lds_per_block &&
        (blocks + dev.cus - 1) / dev.cus <= blocks_per_cu(fn, lds, (int)w * kWave))
      return (int)w;
  }
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
  if (best == 0 && stream && lds_fixed + 8 * lds_per_wave <= dev.lds_per_block) return 8;
  return best;
}

// The one-group-per-wave launch when the row groups fit in the resident
// waves (or stream, for 1-2 tokens) and C is a whole number of lane steps
// with an instantiated count; hipErrorNotSupported when it does not apply
// (the caller then takes the persistent launch).
template <class K, int F, int NT, int LPR, bool XF32, int CPL>
static hipError_t once_launch_t(const DevInfo& dev, typename K::Map map, typename K::Epi epi,
                                const char* x, int64_t ldx_bytes, int C, hipStream_t s,
                                int slices) {
  constexpr int G = kWave / LPR * K::rows_per_team(NT);
  const size_t lds_x = (size_t)NT * C * 16 * ChunkPlanes<F, XF32>::P;
  const size_t lds_wave = (size_t)G * row_scale_pieces(F, C) * 16;  // a wave's scale rows
  const void* fn = once_fn<K, F, NT, LPR, XF32, CPL>();
  const size_t lds_max = std::min(lds_x + kOnceMaxBlock / kWave * lds_wave, dev.lds_per_block);
  if (hipError_t e = allow_dynamic_lds(fn, lds_max)) return e;
  const int64_t n_groups = (K::rows(map) + G - 1) / G;
  const int w = once_waves(dev, fn, n_groups, lds_x, lds_wave, NT <= 2);
  if (w == 0) return hipErrorNotSupported;
  const size_t lds = lds_x + (size_t)w * lds_wave;
  const int64_t blocks = (n_groups + w - 1) / w;
  if constexpr (once_early(NT)) {
    // The early image needs a thread per piece of a token and the same
    // residency (its registers differ slightly from the late kernel's).
    const void* fe = once_fn<K, F, NT, LPR, XF32, CPL, 1>();
    const int64_t per_cu = (blocks + dev.cus - 1) / dev.cus;
    const int res_late = blocks_per_cu(fn, lds, w * kWave);
    const int res_early = blocks_per_cu(fe, lds, w * kWave);
    if ((int64_t)C * ChunkPlanes<F, XF32>::P <= (int64_t)w * kWave &&
        (per_cu <= res_early || per_cu > res_late)) {
      if (hipError_t e = allow_dynamic_lds(fe, lds_max)) return e;
      fn = fe;
    }
  }
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel(fn, dim3((unsigned)blocks, (unsigned)slices), dim3(w * kWave), args, lds,
                         s);
}

template <class K, int F, int NT, int LPR, bool XF32>
static hipError_t once_launch(const DevInfo& dev, const typename K::Map& map,
                              const typename K::Epi& epi, const char* x, int64_t ldx_bytes, int C,
                              hipStream_t s, int slices) {
  if (C % LPR != 0 || slices < 1 || slices > 65535 || (slices > 1 && NT < kMinSliceNT))
    return hipErrorNotSupported;
  switch (C / LPR) {
#define Q8_ONCE(N) \
  case N: return once_launch_t<K, F, NT, LPR, XF32, N>(dev, map, epi, x, ldx_bytes, C, s, slices);
    Q8_ONCE(1) Q8_ONCE(2) Q8_ONCE(3) Q8_ONCE(4) Q8_ONCE(5) Q8_ONCE(6) Q8_ONCE(7) Q8_ONCE(8)
    Q8_ONCE(10) Q8_ONCE(12) Q8_ONCE(14) Q8_ONCE(16)
#undef Q8_ONCE
  }
  return hipErrorNotSupported;
}

template <class K, int NT>
hipError_t launch_once_nt(const DevInfo& dev, const typename K::Map& map,
                          const typename K::Epi& epi, int fmt, int lpr, bool x_f32, const char* x,
                          int64_t ldx_bytes, int C, hipStream_t s, int slices) {
  return dispatch_chunks(fmt, lpr, x_f32, [&](auto f, auto l, auto xf) {
    return once_launch<K, decltype(f)::value, NT, decltype(l)::value, decltype(xf)::value>(
        dev, map, epi, x, ldx_bytes, C, s, slices);
  });
}

// Each (kind, token count) is instantiated in its own translation unit
// (q8_once.hip, built once per pair so the build runs them in parallel);
// everywhere else these instantiations are only declared.
#define Q8_ONCE_DECLARE(KIND, N)                                                              \
  extern template hipError_t launch_once_nt<KIND, N>(const DevInfo&, const KIND::Map&,       \
                                                     const KIND::Epi&, int, int, bool,         \
                                                     const char*, int64_t, int, hipStream_t, \
                                                     int);
#define Q8_ONCE_DECLARE_ALL(KIND)                                                             \
  Q8_ONCE_DECLARE(KIND, 1) Q8_ONCE_DECLARE(KIND, 2) Q8_ONCE_DECLARE(KIND, 3)                  \
  Q8_ONCE_DECLARE(KIND, 4) Q8_ONCE_DECLARE(KIND, 5) Q8_ONCE_DECLARE(KIND, 6)                  \
  Q8_ONCE_DECLARE(KIND, 7) Q8_ONCE_DECLARE(KIND, 8)
Q8_ONCE_DECLARE_ALL(DenseKind)
Q8_ONCE_DECLARE_ALL(GluKind)
#undef Q8_ONCE_DECLARE_ALL
#undef Q8_ONCE_DECLARE

}  // namespace q8
