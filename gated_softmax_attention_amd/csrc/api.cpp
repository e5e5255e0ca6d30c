// C ABI of the FiX attention library: descriptor validation, workspace
// layout and the launch sequence of every entry point declared in
// include/fixattn.h.  Validation is pure host code and makes no HIP call.
#include "fixattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct Shape {
  int64_t Ttot, nseq, nch_ub, nqb_ub;
};

Shape shape_of(const fix_attn_desc *d) {
  Shape s;
  s.Ttot = d->B * d->T;
  s.nseq = d->cu_seqlens ? d->num_seqs : d->B;
  s.nch_ub = cdiv(s.Ttot, fix::CH) + s.nseq;
  s.nqb_ub = cdiv(s.Ttot, fix::QB) + s.nseq;
  return s;
}

// Bump allocator over the caller's workspace (or a null base to measure it).
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *b) : base((char *)b) {}
  template <class T> T *take(int64_t count) {
    size_t at = off;
    off = align_up(off + (size_t)count * sizeof(T));
    return base ? (T *)(base + at) : nullptr;
  }
};

struct FwdWs {
  fix::Plan plan;
  float *Gl2, *Gam;
  _Float16 *VtT;
};

void carve_plan(Carve &cv, const fix_attn_desc *d, const Shape &s, fix::Plan &p) {
  p.seq_start = cv.take<int>(s.nseq);
  p.seq_len = cv.take<int>(s.nseq);
  p.chunk_base = cv.take<int>(s.nseq + 1);
  p.qitems = cv.take<int2>(s.nqb_ub);
  p.counts = cv.take<int>(4);
  p.nseq = (int)s.nseq;
}

size_t carve_fwd(Carve &cv, const fix_attn_desc *d, FwdWs &w) {
  Shape s = shape_of(d);
  carve_plan(cv, d, s, w.plan);
  w.Gl2 = cv.take<float>(s.Ttot * d->Hkv * d->dv);
  w.Gam = cv.take<float>(s.nch_ub * d->Hkv * d->dv);
  w.VtT = cv.take<_Float16>(s.nch_ub * d->Hkv * d->dv * fix::CH);
  return cv.off;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

fix_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return FIX_E_HIP;
}

}  // namespace

extern "C" {

fix_status fix_attn_validate(const fix_attn_desc *d) {
  if (!d) return FIX_E_INVALID;
  if (d->B < 1 || d->T < 1 || d->Hq < 1 || d->Hkv < 1 || d->dk < 1 || d->dv < 1) return FIX_E_INVALID;
  if (d->Hq % d->Hkv != 0) return FIX_E_INVALID;
  if (d->in_dtype != FIX_BF16 && d->in_dtype != FIX_F32) return FIX_E_INVALID;
  if (d->out_dtype != FIX_BF16 && d->out_dtype != FIX_F32) return FIX_E_INVALID;
  if (std::isnan(d->scale) || std::isnan(d->eps) || std::isinf(d->scale) || std::isinf(d->eps) || d->eps < 0)
    return FIX_E_INVALID;
  if (d->cu_seqlens && (d->B != 1 || d->num_seqs < 1)) return FIX_E_INVALID;
  if (!head_dim_ok(d->dk) || !head_dim_ok(d->dv)) return FIX_E_UNSUPPORTED;
  const int64_t Ttot = d->B * d->T;
  if (d->T >= (int64_t(1) << 31) || Ttot >= (int64_t(1) << 31)) return FIX_E_UNSUPPORTED;
  const int64_t H = d->Hq > d->Hkv ? d->Hq : d->Hkv, D = d->dk > d->dv ? d->dk : d->dv;
  if ((double)Ttot * (double)H * (double)D >= (double)(int64_t(1) << 40)) return FIX_E_UNSUPPORTED;
  if (d->cu_seqlens && d->num_seqs >= (int64_t(1) << 24)) return FIX_E_UNSUPPORTED;
  if ((double)shape_of(d).nqb_ub * (double)d->Hq >= 2147483647.0) return FIX_E_UNSUPPORTED;
  return FIX_OK;
}

size_t fix_attn_fwd_workspace_size(const fix_attn_desc *d) {
  if (fix_attn_validate(d) != FIX_OK) return 0;
  Carve cv(nullptr);
  FwdWs w;
  return carve_fwd(cv, d, w);
}

fix_status fix_attn_fwd(const fix_attn_desc *d, const void *q, const void *k, const void *v, const float *g,
                        const void *o_norm_weight, const void *o_gate, void *o, float *m, float *rstd, float *x,
                        void *ws, size_t ws_bytes, void *hip_stream) {
  fix_status stt = fix_attn_validate(d);
  if (stt != FIX_OK) return stt;
  if (!q || !k || !v || !g || !o || !m || !rstd) return FIX_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      (x && !aligned16(x)) || (o_gate && !aligned16(o_gate)))
    return FIX_E_INVALID;
  const size_t need = fix_attn_fwd_workspace_size(d);
  if (ws_bytes < need || (need && !ws)) return FIX_E_WORKSPACE;
  if (!aligned16(ws)) return FIX_E_INVALID;
  hipStream_t st = (hipStream_t)hip_stream;
  Shape s = shape_of(d);
  Carve cv(ws);
  FwdWs w;
  carve_fwd(cv, d, w);
  const bool f32in = d->in_dtype == FIX_F32;
  hipError_t e = fix::launch_plan(d->cu_seqlens, (int)s.nseq, (int)d->T, s.Ttot, w.plan, st);
  if (e != hipSuccess) return hip_fail(e);
  e = fix::launch_gate_prep((int)d->dv, g, v, f32in, w.plan, (int)d->Hkv, (int)s.nch_ub, w.Gl2, w.Gam, w.VtT, st);
  if (e != hipSuccess) return hip_fail(e);
  fix::FwdArgs a;
  a.q = q; a.k = k; a.v = v;
  a.Gl2 = w.Gl2; a.Gam = w.Gam; a.VtT = w.VtT;
  a.w = o_norm_weight; a.z = o_gate;
  a.o = o; a.m = m; a.rstd = rstd; a.x = x;
  a.plan = w.plan;
  a.Hq = (int)d->Hq; a.Hkv = (int)d->Hkv;
  const float scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->dk);
  a.sl2 = scale * fix::LOG2E;
  a.eps = d->eps;
  a.o_norm = d->o_norm ? 1 : 0;
  a.out_f32 = d->out_dtype == FIX_F32;
  e = fix::launch_fwd((int)d->dk, (int)d->dv, f32in, a, (int)(s.nqb_ub * d->Hq), st);
  if (e != hipSuccess) return hip_fail(e);
  return FIX_OK;
}

size_t fix_attn_bwd_workspace_size(const fix_attn_desc *d) {
  if (fix_attn_validate(d) != FIX_OK) return 0;
  return 256;
}

fix_status fix_attn_bwd(const fix_attn_desc *d, const void *q, const void *k, const void *v, const float *g,
                        const void *o_norm_weight, const void *o_gate, const float *m, const float *rstd,
                        const float *x, const void *d_o, void *dq, void *dk, void *dv, float *dg,
                        float *d_o_norm_weight, void *d_o_gate, void *ws, size_t ws_bytes, void *hip_stream) {
  return FIX_E_UNSUPPORTED;
}

const char *fix_attn_status_string(fix_status s) {
  switch (s) {
    case FIX_OK: return "ok";
    case FIX_E_INVALID: return "invalid argument";
    case FIX_E_UNSUPPORTED: return "unsupported shape or head dimension (head dims must be 16, 32, 64 or 128)";
    case FIX_E_WORKSPACE: return "workspace too small";
    case FIX_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int fix_attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
