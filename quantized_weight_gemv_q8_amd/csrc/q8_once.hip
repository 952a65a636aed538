// q8_once.hip -- the one-group-per-wave kernels of one kind and token
// count: the build compiles this file once per pair, with Q8_ONCE_NT (1..8)
// and Q8_ONCE_GLU (0: dense GEMV and pair; 1: gate/up + SiLU pair) set.
#include "q8_once.hpp"

#if !defined(Q8_ONCE_NT) || !defined(Q8_ONCE_GLU)
#error "q8_once.hip is built with -DQ8_ONCE_NT=<1..8> -DQ8_ONCE_GLU=<0|1>"
#endif

namespace q8 {

#if Q8_ONCE_GLU
using OnceKind = GluKind;
#else
using OnceKind = DenseKind;
#endif

template hipError_t launch_once_nt<OnceKind, Q8_ONCE_NT>(const DevInfo&, const OnceKind::Map&,
                                                         const OnceKind::Epi&, int, int, bool,
                                                         const char*, int64_t, int, hipStream_t,
                                                         int);

}  // namespace q8
