// Backward kernel instances with dk = 128 (all dv and input types).
#include "bwd_kernel.h"

namespace fix {
hipError_t launch_bwd_d128(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st) {
  return launch_bwd_dk<128>(kind, dv, f32in, a, grid, st);
}
}  // namespace fix
