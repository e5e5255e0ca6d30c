// Scalar-gate backward kernels for dk = 32 (one translation unit per dk, compiled in parallel).
#include "fox_bwd.h"

namespace fix {
hipError_t launch_fox_bwd_d32(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st) {
  return launch_fox_bwd_dk<32>(kind, dv, a, grid, st);
}
}  // namespace fix
