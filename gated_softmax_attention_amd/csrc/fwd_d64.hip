// Forward kernel instances with dk = 64 (all dv and input types).
#include "fwd_kernel.h"

namespace fix {
hipError_t launch_fwd_d64(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st) {
  return launch_fwd_dk<64>(dv, f32in, a, grid, st);
}
}  // namespace fix
