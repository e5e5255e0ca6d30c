// Scalar-gate backward kernels for dk = 16 (one translation unit per dk, compiled in parallel).
#include "fox_bwd.h"

namespace fix {
hipError_t launch_fox_bwd_d16(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st) {
  return launch_fox_bwd_dk<16>(kind, dv, a, grid, st);
}
}  // namespace fix
