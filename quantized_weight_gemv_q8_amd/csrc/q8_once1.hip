// q8_once1.hip -- one-group-per-wave dense GEMV kernels for 1-token passes.
#include "q8_once.hpp"

namespace q8 {

hipError_t launch_once_nt1(const DevInfo& dev, const DenseMap& map, const DenseEpi& epi, int fmt,
                             int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                             hipStream_t s) {
  return launch_once_nt<DenseKind, 1>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
}

hipError_t launch_gemv_once(int nt, const DevInfo& dev, const DenseMap& map, const DenseEpi& epi,
                            int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                            hipStream_t s) {
  switch (nt) {
    case 1: return launch_once_nt1(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 2: return launch_once_nt2(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 3: return launch_once_nt3(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 4: return launch_once_nt4(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 5: return launch_once_nt5(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 6: return launch_once_nt6(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 7: return launch_once_nt7(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 8: return launch_once_nt8(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
  }
  return hipErrorNotSupported;
}

hipError_t launch_glu_once_nt1(const DevInfo& dev, const GluMap& map, const GluEpi& epi, int fmt,
                              int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                              hipStream_t s) {
  return launch_once_nt<GluKind, 1>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
}

hipError_t launch_glu_once(int nt, const DevInfo& dev, const GluMap& map, const GluEpi& epi,
                           int fmt, int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                           hipStream_t s) {
  switch (nt) {
    case 1: return launch_glu_once_nt1(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 2: return launch_glu_once_nt2(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 3: return launch_glu_once_nt3(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 4: return launch_glu_once_nt4(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 5: return launch_glu_once_nt5(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 6: return launch_glu_once_nt6(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 7: return launch_glu_once_nt7(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
    case 8: return launch_glu_once_nt8(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
  }
  return hipErrorNotSupported;
}

}  // namespace q8
