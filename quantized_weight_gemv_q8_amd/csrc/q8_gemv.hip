// q8_gemv.hip -- dense Q8_0 GEMV and the fused gate+up pair (gfx950).
//
// One persistent launch per pass of up to 8 tokens. Workgroups stage x
// into LDS once, then their waves walk row groups with a grid stride, so
// every weight byte is fetched from HBM exactly once per pass and x is
// reused from LDS for all rows (memra wiki, feature list: Q8_0 decode
// matvecs with per-shape auto-dispatch; here the shape picks the lanes per
// row and the token count picks the rows per team).
#include "q8_engine.hpp"
#include "q8_internal.h"

namespace q8 {

struct DenseMap {
  MatDesc a, b;
  int64_t Ma, Mtot;
  __device__ __forceinline__ bool row(int64_t i, const int8_t*& q, const uint16_t*& d) const {
    q = a.qs;
    d = a.d;
    if (i >= Mtot) return false;
    if (i < Ma) {
      q = a.qs + i * a.ld_qs;
      d = a.d + i * a.ld_d;
    } else {
      const int64_t k = i - Ma;
      q = b.qs + k * b.ld_qs;
      d = b.d + k * b.ld_d;
    }
    return true;
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

template <int NT>
struct RowsPerTeam {
  static constexpr int value = NT <= 2 ? 2 : 4;
};

template <int NT, int LPR, bool XF32>
__global__ __launch_bounds__(kBlock) void gemv_kernel(DenseMap map, DenseEpi epi, const char* x,
                                                      int64_t ldx_bytes, int C) {
  extern __shared__ uint4 lds_x[];
  constexpr int R = RowsPerTeam<NT>::value;
  constexpr int G = (kWave / LPR) * R;
  const char* rows[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) rows[n] = x + n * ldx_bytes;
  stage_x<NT, XF32>(rows, C, lds_x);
  __syncthreads();
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int wave = threadIdx.x / kWave;
  run_rows<NT, LPR, R, 1, XF32>(map, epi, lds_x, C, n_groups,
                                (int64_t)blockIdx.x * kWavesPerBlock + wave,
                                (int64_t)gridDim.x * kWavesPerBlock, 0);
}

template <int NT, int LPR, bool XF32>
static hipError_t launch_t(const DevInfo& dev, DenseMap map, DenseEpi epi, const char* x,
                           int64_t ldx_bytes, int C, hipStream_t s) {
  constexpr int R = RowsPerTeam<NT>::value;
  constexpr int G = (kWave / LPR) * R;
  const size_t lds = (size_t)NT * C * 16 * XPlanes<XF32>::P;
  const int64_t n_groups = (map.Mtot + G - 1) / G;
  const int64_t need = (n_groups + kWavesPerBlock - 1) / kWavesPerBlock;
  int64_t per_cu = lds ? (int64_t)(160 * 1024 / lds) : 4;
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 4) per_cu = 4;
  int64_t blocks = (int64_t)dev.cus * per_cu;
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  auto fn = gemv_kernel<NT, LPR, XF32>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&map, &epi, (void*)&x, &ldx_bytes, &C};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)blocks), dim3(kBlock), args, lds, s);
}

template <int LPR, bool XF32>
static hipError_t launch_nt(const DevInfo& dev, int nt, DenseMap map, DenseEpi epi, const char* x,
                            int64_t ldx_bytes, int C, hipStream_t s) {
  switch (nt) {
    case 1: return launch_t<1, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 2: return launch_t<2, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 3: return launch_t<3, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 4: return launch_t<4, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 5: return launch_t<5, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 6: return launch_t<6, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 7: return launch_t<7, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
    case 8: return launch_t<8, LPR, XF32>(dev, map, epi, x, ldx_bytes, C, s);
  }
  return hipErrorInvalidValue;
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
  map.a = MatDesc{A.qs, A.d, A.ld_qs, A.ld_d};
  map.b = B ? MatDesc{B->qs, B->d, B->ld_qs, B->ld_d} : map.a;
  map.Ma = A.M;
  map.Mtot = A.M + (B ? B->M : 0);
  DenseEpi epi;
  epi.ya = (char*)ya;
  epi.yb = (char*)yb;
  epi.Ma = map.Ma;
  epi.Mtot = map.Mtot;
  epi.f16 = y_f16;
  const int C = (int)(A.K / 16);
  const int64_t ldx_bytes = ldx * (x_f32 ? 4 : 2);
  const char* xp = (const char*)x;
  const int lpr = lanes_per_row(A.K);
  if (x_f32) {
    if (lpr == 64) return launch_nt<64, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
    if (lpr == 32) return launch_nt<32, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
    return launch_nt<16, true>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  }
  if (lpr == 64) return launch_nt<64, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  if (lpr == 32) return launch_nt<32, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
  return launch_nt<16, false>(dev, nt, map, epi, xp, ldx_bytes, C, s);
}

}  // namespace q8
