// Host-side launchers exported by each kernel translation unit.
#pragma once
#include <hip/hip_runtime.h>

#include "common.h"

namespace fix {

struct FwdArgs {
  const void *q, *k, *v;
  const float *Gl2, *Gam;
  const _Float16 *VtT;
  const void *w, *z;
  void *o;
  float *m, *rstd, *x;
  Plan plan;
  int Hq, Hkv;
  float sl2;  // softmax scale * log2(e)
  float eps;
  int o_norm;
  int out_f32;
};

hipError_t launch_plan(const int64_t *cu, int nseq, int T, int64_t Ttot, const Plan &plan, hipStream_t st);
hipError_t launch_gate_prep(int dv, const float *g, const void *v, bool in_f32, const Plan &plan, int Hkv,
                            int nch_ub, float *Gl2, float *Gam, _Float16 *VtT, hipStream_t st);
hipError_t launch_fwd_d16(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fwd_d32(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fwd_d64(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fwd_d128(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st);

inline hipError_t launch_fwd(int dk, int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st) {
  switch (dk) {
    case 16: return launch_fwd_d16(dv, f32in, a, grid, st);
    case 32: return launch_fwd_d32(dv, f32in, a, grid, st);
    case 64: return launch_fwd_d64(dv, f32in, a, grid, st);
    case 128: return launch_fwd_d128(dv, f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fix
