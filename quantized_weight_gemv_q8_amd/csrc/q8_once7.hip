// q8_once7.hip -- one-group-per-wave dense GEMV and SiLU-pair kernels for 7-token passes.
#include "q8_once.hpp"

namespace q8 {

hipError_t launch_once_nt7(const DevInfo& dev, const DenseMap& map, const DenseEpi& epi, int fmt,
                             int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                             hipStream_t s) {
  return launch_once_nt<DenseKind, 7>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
}

hipError_t launch_glu_once_nt7(const DevInfo& dev, const GluMap& map, const GluEpi& epi, int fmt,
                              int lpr, bool x_f32, const char* x, int64_t ldx_bytes, int C,
                              hipStream_t s) {
  return launch_once_nt<GluKind, 7>(dev, map, epi, fmt, lpr, x_f32, x, ldx_bytes, C, s);
}

}  // namespace q8
