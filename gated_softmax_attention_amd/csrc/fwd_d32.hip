// Forward kernel instances with dk = 32 (all dv and input types).
#include "fwd_kernel.h"

namespace fix {
hipError_t launch_fwd_d32(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st) {
  return launch_fwd_dk<32>(dv, f32in, a, grid, st);
}
}  // namespace fix
