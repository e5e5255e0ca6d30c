// C ABI of the FiX attention library: descriptor validation, workspace
// layout and the launch sequence of every entry point declared in
// include/fixattn.h.  Validation is pure host code and makes no HIP call.
#include "fixattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

// Opt-in event trace (see fix_attn_set_event_trace).
struct Trace {
  hipEvent_t *events = nullptr;
  int capacity = 0, count = 0;
  const char *labels[64] = {};
};
thread_local Trace g_trace;

// Opt-in launch log: with FIX_ATTN_LOG set in the environment (to anything
// but "0"), each kernel an entry point enqueues writes one line to stderr.
bool launch_log() {
  static const bool on = [] {
    const char *v = std::getenv("FIX_ATTN_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}
thread_local const char *g_entry = "";

hipError_t trace_begin(hipStream_t st, const char *entry) {
  g_entry = entry;
  g_trace.count = 0;
  if (!g_trace.events || g_trace.capacity < 1) return hipSuccess;
  g_trace.labels[0] = "begin";
  g_trace.count = 1;
  return hipEventRecord(g_trace.events[0], st);
}
hipError_t trace_mark(hipStream_t st, const char *label) {
  if (launch_log()) std::fprintf(stderr, "[fixattn] %s: %s enqueued on stream %p\n", g_entry, label, (void *)st);
  if (!g_trace.events || g_trace.count >= g_trace.capacity || g_trace.count >= 64) return hipSuccess;
  g_trace.labels[g_trace.count] = label;
  return hipEventRecord(g_trace.events[g_trace.count++], st);
}

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
  float *Gl2 = nullptr, *Gam = nullptr;
  _Float16 *VtT = nullptr;
  // scalar gate: v as fp16, the gate's block-local prefix and block references
  _Float16 *V16 = nullptr;
  float *loc = nullptr;
  double *ref = nullptr;
};

void carve_plan(Carve &cv, const fix_attn_desc *d, const Shape &s, fix::Plan &p) {
  p.seq_start = cv.take<int>(s.nseq);
  p.seq_len = cv.take<int>(s.nseq);
  p.chunk_base = cv.take<int>(s.nseq + 1);
  p.cb128 = cv.take<int>(s.nseq + 1);
  p.counts = cv.take<int>(4);
  p.nseq = (int)s.nseq;
}

size_t carve_fwd(Carve &cv, const fix_attn_desc *d, FwdWs &w) {
  Shape s = shape_of(d);
  carve_plan(cv, d, s, w.plan);
  if (d->gate_scalar) {
    w.V16 = cv.take<_Float16>(s.Ttot * d->Hkv * d->dv);
    w.loc = cv.take<float>(s.Ttot * d->Hkv);
    w.ref = cv.take<double>(s.nch_ub * d->Hkv);
    return cv.off;
  }
  w.Gl2 = cv.take<float>(s.Ttot * d->Hkv * d->dv);
  w.Gam = cv.take<float>(s.nch_ub * d->Hkv * d->dv);
  w.VtT = cv.take<_Float16>(s.nch_ub * d->Hkv * d->dv * fix::CH);
  return cv.off;
}

struct BwdWs {
  fix::Plan plan;
  float *Gl2, *Gam;
  double *Lam;
  _Float16 *Vr, *Kt, *VE, *Q16;
  __bf16 *VBH, *VBL;
  float *prj;
  _Float16 *dh, *dhT, *X16;
  __bf16 *XH, *XL;
  float *mb, *sig, *qside, *dG, *dq_i, *dk_i, *dv_i, *dw_part, *dg_tot, *dg_carry;
};

// Scalar-gate backward workspace (logit-bias form; fox_bwd.h).
struct FoxBwdWs {
  fix::Plan plan;
  float *loc;
  double *ref;
  _Float16 *Q16, *K16, *V16, *D16;
  float *mb, *rsum, *csum, *dw_part;
};

int64_t pad32(int64_t d) { return d < 32 ? 32 : d; }

size_t carve_fox_bwd(Carve &cv, const fix_attn_desc *d, FoxBwdWs &w) {
  Shape s = shape_of(d);
  carve_plan(cv, d, s, w.plan);
  const int64_t T = s.Ttot, Hq = d->Hq, Hkv = d->Hkv;
  w.loc = cv.take<float>(T * Hkv);
  w.ref = cv.take<double>(s.nch_ub * Hkv);
  w.Q16 = cv.take<_Float16>(T * Hq * pad32(d->dk));
  w.K16 = cv.take<_Float16>(T * Hkv * pad32(d->dk));
  w.V16 = cv.take<_Float16>(T * Hkv * d->dv);
  w.D16 = cv.take<_Float16>(T * Hq * pad32(d->dv));
  w.mb = cv.take<float>(T * Hq);
  w.rsum = cv.take<float>(T * Hq);
  w.csum = cv.take<float>(T * Hkv);
  w.dw_part = cv.take<float>(s.nqb_ub * Hkv * d->dv);
  return cv.off;
}

size_t carve_bwd(Carve &cv, const fix_attn_desc *d, BwdWs &w) {
  Shape s = shape_of(d);
  carve_plan(cv, d, s, w.plan);
  const int64_t T = s.Ttot, ncb = s.nqb_ub, Hq = d->Hq, Hkv = d->Hkv, DK = d->dk, DV = d->dv;
  w.Gl2 = cv.take<float>(T * Hkv * DV);
  w.Gam = cv.take<float>(ncb * Hkv * DV);
  w.Lam = cv.take<double>(ncb * Hkv * DV);
  w.Vr = cv.take<_Float16>(ncb * Hkv * fix::CB * DV);
  w.Q16 = cv.take<_Float16>(T * Hq * DK);
  w.Kt = cv.take<_Float16>(ncb * Hkv * DK * fix::CB);
  w.prj = cv.take<float>(T * Hq);
  w.dh = cv.take<_Float16>(T * Hq * DV);
  w.dhT = cv.take<_Float16>(ncb * Hq * DV * fix::CB);
  w.VE = cv.take<_Float16>(T * Hkv * DV);
  w.VBH = cv.take<__bf16>(T * Hkv * DV);
  w.VBL = cv.take<__bf16>(T * Hkv * DV);
  w.X16 = cv.take<_Float16>(T * Hq * DV);
  w.XH = cv.take<__bf16>(T * Hq * DV);
  w.XL = cv.take<__bf16>(T * Hq * DV);
  w.mb = cv.take<float>(T * Hq);
  w.sig = cv.take<float>(T * Hq);
  w.qside = cv.take<float>(T * Hkv * DV);
  w.dG = cv.take<float>(T * Hkv * DV);
  w.dq_i = cv.take<float>(T * Hq * DK);
  w.dk_i = cv.take<float>(T * Hkv * DK);
  w.dv_i = cv.take<float>(T * Hkv * DV);
  w.dw_part = cv.take<float>(ncb * Hkv * DV);
  w.dg_tot = cv.take<float>(ncb * Hkv * 4 * DV);
  w.dg_carry = cv.take<float>(ncb * Hkv * DV);
  return cv.off;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Grids of kernels that order their work per XCD hold a multiple of 8 workgroups.
int64_t round8(int64_t n) { return (n + 7) / 8 * 8; }

fix_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return FIX_E_HIP;
}

}  // namespace

// ---- decode cache and workspace layout (see decode.hip) ----
int decode_splits(const fix_decode_desc *d) {
  // 16 chunks per split: measured best at T = 8192 (fewer add per-workgroup
  // cost, more leave too few workgroups)
  const int64_t nch = d->cap / fix::CH, s = cdiv(nch, 16);
  return (int)(s < 1 ? 1 : s > 64 ? 64 : s);
}
size_t carve_decode(Carve &cv, const fix_decode_desc *d, fix::DecodeCache &dc) {
  const int64_t B = d->B, cap = d->cap, Hkv = d->Hkv, nch = cap / fix::CH;
  dc.B = (int)B; dc.cap = (int)cap; dc.Hq = (int)d->Hq; dc.Hkv = (int)Hkv; dc.G = (int)(d->Hq / d->Hkv);
  dc.dk = (int)d->dk; dc.dv = (int)d->dv;
  dc.len = cv.take<int>(B);
  dc.K = cv.take<_Float16>(B * cap * Hkv * d->dk);
  dc.VT = cv.take<_Float16>(B * nch * Hkv * d->dv * fix::CH);
  dc.Vo = cv.take<_Float16>(B * fix::CH * Hkv * d->dv);
  dc.Go = cv.take<float>(B * fix::CH * Hkv * d->dv);
  dc.Lam = cv.take<double>(B * (nch + 1) * Hkv * d->dv);
  return cv.off;
}
struct DecodeWs {
  float *part, *mpart;
  _Float16 *vto;  // the open chunk of every (sequence, kv head), decayed to the newest token
};
size_t carve_decode_ws(Carve &cv, const fix_decode_desc *d, DecodeWs &w) {
  const int64_t units = 4 * decode_splits(d), rows = d->B * d->Hkv * units * (d->Hq / d->Hkv);
  w.part = cv.take<float>(rows * d->dv);
  w.mpart = cv.take<float>(rows);
  w.vto = cv.take<_Float16>(d->B * d->Hkv * d->dv * fix::CH);
  return cv.off;
}

// ---- scratch of the allocation-free decode step ----
// One copy of this array lives on every GPU the library runs on; host code
// must never pass its name to a kernel (that is a host-side stand-in): the
// device address of each GPU's copy is resolved once per device and kept.
static __device__ __align__(256) char scratch[FIX_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of the scratch array.
hipError_t decode_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
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
  if (d->gate_scalar != 0 && d->gate_scalar != 1) return FIX_E_INVALID;
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
  hipError_t e = trace_begin(st, "fix_attn_fwd");
  if (e != hipSuccess) return hip_fail(e);
  e = fix::launch_plan(d->cu_seqlens, (int)s.nseq, (int)d->T, s.Ttot, w.plan, st);
  if (e == hipSuccess) e = trace_mark(st, "plan");
  if (e != hipSuccess) return hip_fail(e);
  if (d->gate_scalar) {  // decay as a logit bias: no value scaling
    const float scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->dk);
    e = fix::launch_fox_prefix(g, d->gate_logits != 0, w.plan, (int)s.nseq, (int)d->Hkv, w.loc, w.ref, st);
    if (e == hipSuccess) e = trace_mark(st, "fox_prefix");
    if (e == hipSuccess) e = fix::launch_to_f16(v, f32in, s.Ttot * d->Hkv * d->dv, w.V16, st);
    if (e == hipSuccess) e = trace_mark(st, "v_f16");
    if (e != hipSuccess) return hip_fail(e);
    fix::FoxArgs fa;
    fa.q = q; fa.k = k; fa.V16 = w.V16; fa.loc = w.loc; fa.ref = w.ref;
    fa.w = o_norm_weight; fa.z = o_gate;
    fa.o = o; fa.m = m; fa.rstd = rstd; fa.x = x;
    fa.plan = w.plan;
    fa.Hq = (int)d->Hq; fa.Hkv = (int)d->Hkv;
    fa.sl2 = scale * fix::LOG2E;
    fa.eps = d->eps;
    fa.o_norm = d->o_norm ? 1 : 0;
    fa.out_f32 = d->out_dtype == FIX_F32;
    e = fix::launch_fox_fwd((int)d->dk, (int)d->dv, f32in, fa, (int)round8(s.nqb_ub * d->Hq), st);
    if (e == hipSuccess) e = trace_mark(st, "fox_fwd");
    return e == hipSuccess ? FIX_OK : hip_fail(e);
  }
  e = fix::launch_gate_prep((int)d->dv, g, d->gate_logits != 0, v, f32in, w.plan, (int)d->Hkv, (int)s.nch_ub, w.Gl2,
                            w.Gam, w.VtT, st);
  if (e == hipSuccess) e = trace_mark(st, "gate_prep");
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
  e = fix::launch_fwd((int)d->dk, (int)d->dv, f32in, a, (int)round8(s.nqb_ub * d->Hq), st);
  if (e == hipSuccess) e = trace_mark(st, "fix_fwd");
  if (e != hipSuccess) return hip_fail(e);
  return FIX_OK;
}

size_t fix_attn_bwd_workspace_size(const fix_attn_desc *d) {
  if (fix_attn_validate(d) != FIX_OK) return 0;
  Carve cv(nullptr);
  if (d->gate_scalar) {
    FoxBwdWs w;
    return carve_fox_bwd(cv, d, w);
  }
  BwdWs w;
  return carve_bwd(cv, d, w);
}

fix_status fix_attn_bwd(const fix_attn_desc *d, const void *q, const void *k, const void *v, const float *g,
                        const void *o_norm_weight, const void *o_gate, const float *m, const float *rstd,
                        const float *x, const void *d_o, void *dq, void *dk, void *dv, float *dg,
                        float *d_o_norm_weight, void *d_o_gate, void *ws, size_t ws_bytes, void *hip_stream) {
  fix_status stt = fix_attn_validate(d);
  if (stt != FIX_OK) return stt;
  if (!q || !k || !v || !g || !m || !rstd || !x || !d_o || !dq || !dk || !dv || !dg) return FIX_E_INVALID;
  if (d_o_gate && !o_gate) return FIX_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(x) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg) || (o_gate && !aligned16(o_gate)))
    return FIX_E_INVALID;
  const size_t need = fix_attn_bwd_workspace_size(d);
  if (ws_bytes < need || (need && !ws)) return FIX_E_WORKSPACE;
  if (!aligned16(ws)) return FIX_E_INVALID;
  hipStream_t st = (hipStream_t)hip_stream;
  Shape s = shape_of(d);
  const bool f32in = d->in_dtype == FIX_F32;
  const int Hq = (int)d->Hq, Hkv = (int)d->Hkv, DK = (int)d->dk, DV = (int)d->dv, ncb = (int)s.nqb_ub;
  const bool want_dw = d->o_norm && d_o_norm_weight;
  const float scale = d->scale > 0.f ? d->scale : 1.f / std::sqrt((float)d->dk);
  hipError_t e;
#define FIX_TRY(call, label)                        \
  do {                                              \
    e = (call);                                     \
    if (e == hipSuccess) e = trace_mark(st, label); \
    if (e != hipSuccess) return hip_fail(e);        \
  } while (0)
  e = trace_begin(st, "fix_attn_bwd");
  if (e != hipSuccess) return hip_fail(e);
  if (d->gate_scalar) {
    // The decay as a logit bias (fox_bwd.h): dq with the row sums of dS, dk and
    // dv with its column sums, and dg as the suffix sum of their difference.
    Carve cv(ws);
    FoxBwdWs w;
    carve_fox_bwd(cv, d, w);
    const int DKP = (int)pad32(DK), DVP = (int)pad32(DV);
    FIX_TRY(fix::launch_plan(d->cu_seqlens, (int)s.nseq, (int)d->T, s.Ttot, w.plan, st), "plan");
    FIX_TRY(fix::launch_fox_prefix(g, d->gate_logits != 0, w.plan, (int)s.nseq, Hkv, w.loc, w.ref, st), "fox_prefix");
    FIX_TRY(fix::launch_to_f16_pad(q, f32in, s.Ttot * Hq, DK, DKP, w.Q16, st), "q_f16");
    FIX_TRY(fix::launch_to_f16_pad(k, f32in, s.Ttot * Hkv, DK, DKP, w.K16, st), "k_f16");
    FIX_TRY(fix::launch_to_f16(v, f32in, s.Ttot * Hkv * DV, w.V16, st), "v_f16");
    fix::FoxPrepArgs pa;
    pa.x = x; pa.rstd = rstd; pa.m = m;
    pa.dO = d_o; pa.z = o_gate; pa.w = d->o_norm ? o_norm_weight : nullptr;
    pa.plan = w.plan;
    pa.Hq = Hq; pa.Hkv = Hkv;
    pa.o_norm = d->o_norm ? 1 : 0;
    pa.out_f32 = d->out_dtype == FIX_F32;
    pa.in_f32 = f32in;
    pa.D16 = w.D16; pa.mb = w.mb; pa.dz = d_o_gate;
    pa.dw_part = want_dw ? w.dw_part : nullptr;
    FIX_TRY(fix::launch_fox_bwd_prep(DV, pa, ncb, st), "fox_bwd_prep");
    fix::FoxBwdArgs fa;
    fa.Q16 = w.Q16; fa.K16 = w.K16; fa.V16 = w.V16; fa.D16 = w.D16;
    fa.mb = w.mb; fa.loc = w.loc; fa.ref = w.ref; fa.rsum = w.rsum; fa.csum = w.csum;
    fa.dq = dq; fa.dk = dk; fa.dv = dv;
    fa.plan = w.plan;
    fa.Hq = Hq; fa.Hkv = Hkv;
    fa.sl2 = scale * fix::LOG2E;
    fa.scale = scale;
    fa.out_f32 = d->out_dtype == FIX_F32;
    FIX_TRY(fix::launch_fox_bwd(fix::FK_DQ, DK, DV, fa, (int)round8(s.nqb_ub * Hq), st), "fox_bwd_dq");
    FIX_TRY(fix::launch_fox_bwd(fix::FK_DKV, DK, DV, fa, (int)round8(s.nqb_ub * Hkv), st), "fox_bwd_dkv");
    FIX_TRY(fix::launch_fox_dg_scan(w.rsum, w.csum, d->gate_logits ? g : nullptr, w.plan, (int)s.nseq, Hq, Hkv, dg, st),
            "fox_dg_scan");
    if (want_dw) FIX_TRY(fix::launch_dw_reduce(w.dw_part, w.plan.counts, Hkv, DV, d_o_norm_weight, st), "dw_reduce");
    return FIX_OK;
  }
  Carve cv(ws);
  BwdWs w;
  carve_bwd(cv, d, w);
  FIX_TRY(fix::launch_plan(d->cu_seqlens, (int)s.nseq, (int)d->T, s.Ttot, w.plan, st), "plan");
  FIX_TRY(fix::launch_gate_prep_rows(DV, g, d->gate_logits != 0, v, f32in, w.plan, Hkv, ncb, w.Gl2, w.Gam, w.Vr,
                                     w.VE, w.VBH, w.VBL, st),
          "gate_prep_rows");
  FIX_TRY(fix::launch_chunk_logprefix(DV, w.Gl2, w.plan, Hkv, w.Lam, st), "chunk_logprefix");
  FIX_TRY(fix::launch_tiles_t(DK, k, f32in, w.plan, Hkv, ncb, w.Kt, st), "tiles_k");
  FIX_TRY(fix::launch_to_f16(q, f32in, s.Ttot * Hq * DK, w.Q16, st), "q_f16");
  fix::PrepArgs pa;
  pa.x = x; pa.rstd = rstd; pa.m = m; pa.Gl2 = w.Gl2;
  pa.dO = d_o; pa.z = o_gate; pa.w = d->o_norm ? o_norm_weight : nullptr;
  pa.plan = w.plan;
  pa.Hq = Hq; pa.Hkv = Hkv;
  pa.o_norm = d->o_norm ? 1 : 0;
  pa.out_f32 = d->out_dtype == FIX_F32;
  pa.in_f32 = f32in;
  pa.prj = w.prj; pa.dh = w.dh; pa.mb = w.mb; pa.sig = w.sig; pa.qside = w.qside;
  pa.dz = d_o_gate;
  pa.X16 = w.X16; pa.XH = w.XH; pa.XL = w.XL;
  pa.dw_part = want_dw ? w.dw_part : nullptr;
  FIX_TRY(fix::launch_bwd_prep(DV, pa, ncb, st), "bwd_prep");
  FIX_TRY(fix::launch_tiles_t(DV, w.dh, 2, w.plan, Hq, ncb, w.dhT, st), "tiles_dh");
  fix::BwdArgs a;
  a.q = q; a.k = k; a.v = v;
  a.Gl2 = w.Gl2; a.Gam = w.Gam; a.Lam = w.Lam; a.Vr = w.Vr; a.Kt = w.Kt; a.Q16 = w.Q16;
  a.x = x; a.rstd = rstd; a.prj = w.prj; a.dO = d_o; a.z = o_gate; a.w = d->o_norm ? o_norm_weight : nullptr;
  a.o_norm = d->o_norm ? 1 : 0;
  a.dh = w.dh; a.dhT = w.dhT; a.mb = w.mb; a.sig = w.sig; a.qside = w.qside;
  a.VE = w.VE; a.VBH = w.VBH; a.VBL = w.VBL; a.X16 = w.X16; a.XH = w.XH; a.XL = w.XL;
  a.dq_i = w.dq_i; a.dk_i = w.dk_i; a.dv_i = w.dv_i;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dG = w.dG; a.dg_tot = w.dg_tot;
  a.plan = w.plan;
  a.Hq = Hq; a.Hkv = Hkv;
  a.sl2 = scale * fix::LOG2E;
  a.scale = scale;
  a.out_f32 = d->out_dtype == FIX_F32;
  FIX_TRY(fix::launch_bwd(fix::BK_INTRA_DQ, DK, DV, f32in, a, dim3(ncb, Hq), st), "bwd_intra_dq");
  FIX_TRY(fix::launch_bwd(fix::BK_INTRA_DKV, DK, DV, f32in, a, dim3(ncb, Hkv), st), "bwd_intra_dkv");
  FIX_TRY(fix::launch_bwd(fix::BK_DQ, DK, DV, f32in, a, dim3(round8(ncb * Hq)), st), "bwd_dq");
  FIX_TRY(fix::launch_bwd(fix::BK_DKV, DK, DV, f32in, a, dim3(round8(ncb * Hkv)), st), "bwd_dkv");
  FIX_TRY(fix::launch_dg_scan(DV, w.dG, d->gate_logits ? g : nullptr, w.plan, Hkv, ncb, w.dg_tot, w.dg_carry, dg,
                              st),
          "dg_scan");
  if (want_dw) {
    FIX_TRY(fix::launch_dw_reduce(w.dw_part, w.plan.counts, Hkv, DV, d_o_norm_weight, st), "dw_reduce");
  }
#undef FIX_TRY
  return FIX_OK;
}

fix_status fix_decode_validate(const fix_decode_desc *d) {
  if (!d) return FIX_E_INVALID;
  if (d->B < 1 || d->cap < 1 || d->Hq < 1 || d->Hkv < 1 || d->dk < 1 || d->dv < 1) return FIX_E_INVALID;
  if (d->Hq % d->Hkv != 0 || d->cap % fix::CH != 0) return FIX_E_INVALID;
  if (d->in_dtype != FIX_BF16 && d->in_dtype != FIX_F32) return FIX_E_INVALID;
  if (d->out_dtype != FIX_BF16 && d->out_dtype != FIX_F32) return FIX_E_INVALID;
  if (std::isnan(d->scale) || std::isnan(d->eps) || std::isinf(d->scale) || std::isinf(d->eps) || d->eps < 0)
    return FIX_E_INVALID;
  if (!head_dim_ok(d->dk) || !head_dim_ok(d->dv)) return FIX_E_UNSUPPORTED;
  if (d->Hq / d->Hkv > 32) return FIX_E_UNSUPPORTED;
  if (d->cap >= (int64_t(1) << 30) || d->B >= (int64_t(1) << 20) || d->B * d->Hq >= (int64_t(1) << 31))
    return FIX_E_UNSUPPORTED;
  const int64_t D = d->dk > d->dv ? d->dk : d->dv;
  if ((double)d->B * (double)d->cap * (double)d->Hkv * (double)D >= (double)(int64_t(1) << 40))
    return FIX_E_UNSUPPORTED;
  return FIX_OK;
}

size_t fix_decode_cache_size(const fix_decode_desc *d) {
  if (fix_decode_validate(d) != FIX_OK) return 0;
  Carve cv(nullptr);
  fix::DecodeCache dc;
  return carve_decode(cv, d, dc);
}

size_t fix_decode_workspace_size(const fix_decode_desc *d) {
  if (fix_decode_validate(d) != FIX_OK) return 0;
  Carve cv(nullptr);
  DecodeWs w;
  return carve_decode_ws(cv, d, w);
}

fix_status fix_decode_reset(const fix_decode_desc *d, void *cache, void *hip_stream) {
  fix_status stt = fix_decode_validate(d);
  if (stt != FIX_OK) return stt;
  if (!cache || ((uintptr_t)cache & 255)) return FIX_E_INVALID;
  Carve cv(cache);
  fix::DecodeCache dc;
  carve_decode(cv, d, dc);
  hipError_t e = fix::launch_decode_reset(dc, (hipStream_t)hip_stream);
  return e == hipSuccess ? FIX_OK : hip_fail(e);
}

fix_status fix_decode_append(const fix_decode_desc *d, void *cache, const void *k, const void *v, const float *g,
                             int64_t n, const int32_t *n_seq, void *hip_stream) {
  fix_status stt = fix_decode_validate(d);
  if (stt != FIX_OK) return stt;
  if (!cache || ((uintptr_t)cache & 255) || !k || !v || !g || n < 1 || n > d->cap) return FIX_E_INVALID;
  if (!aligned16(k) || !aligned16(v) || !aligned16(g)) return FIX_E_INVALID;
  Carve cv(cache);
  fix::DecodeCache dc;
  carve_decode(cv, d, dc);
  hipError_t e = fix::launch_decode_append(dc, k, v, g, (int)n, n_seq, d->in_dtype == FIX_F32, d->gate_logits != 0,
                                           (hipStream_t)hip_stream);
  return e == hipSuccess ? FIX_OK : hip_fail(e);
}

fix_status fix_decode_step(const fix_decode_desc *d, const void *cache, const void *q, const void *o_norm_weight,
                           const void *o_gate, void *o, float *m, void *ws, size_t ws_bytes, void *hip_stream) {
  fix_status stt = fix_decode_validate(d);
  if (stt != FIX_OK) return stt;
  if (!cache || ((uintptr_t)cache & 255) || !q || !o) return FIX_E_INVALID;
  if (!aligned16(q) || !aligned16(o) || (o_gate && !aligned16(o_gate))) return FIX_E_INVALID;
  const size_t need = fix_decode_workspace_size(d);
  if (ws_bytes < need || !ws) return FIX_E_WORKSPACE;
  if (!aligned16(ws)) return FIX_E_INVALID;
  hipStream_t st = (hipStream_t)hip_stream;
  Carve cv((void *)cache);
  fix::DecodeCache dc;
  carve_decode(cv, d, dc);
  Carve cw(ws);
  DecodeWs w;
  carve_decode_ws(cw, d, w);
  const bool f32in = d->in_dtype == FIX_F32;
  const float scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  const int splits = decode_splits(d);
  hipError_t e = trace_begin(st, "fix_decode_step");
  if (e == hipSuccess) e = fix::launch_decode_open(dc, w.vto, st);
  if (e == hipSuccess) e = trace_mark(st, "decode_open");
  if (e == hipSuccess) e = fix::launch_decode_step(dc, q, f32in, scale * fix::LOG2E, splits, w.vto, w.part, w.mpart, st);
  if (e == hipSuccess) e = trace_mark(st, "decode_step");
  if (e == hipSuccess)
    e = fix::launch_decode_combine(dc, 4 * splits, w.part, w.mpart, d->o_norm ? o_norm_weight : nullptr, o_gate, f32in,
                                   d->out_dtype == FIX_F32, d->o_norm != 0, d->eps, o, m, st);
  if (e == hipSuccess) e = trace_mark(st, "decode_combine");
  return e == hipSuccess ? FIX_OK : hip_fail(e);
}

fix_status fix_decode_step_noalloc(const fix_decode_desc *d, const void *cache, const void *q,
                                   const void *o_norm_weight, const void *o_gate, void *o, float *m,
                                   void *hip_stream) {
  fix_status stt = fix_decode_validate(d);
  if (stt != FIX_OK) return stt;
  if (fix_decode_workspace_size(d) > FIX_DECODE_SCRATCH_BYTES) return FIX_E_WORKSPACE;
  void *ws = nullptr;
  hipError_t e = decode_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e);
  // every byte of the step's scratch is written before it is read: nothing to clear
  return fix_decode_step(d, cache, q, o_norm_weight, o_gate, o, m, ws, FIX_DECODE_SCRATCH_BYTES, hip_stream);
}

fix_status fix_attn_check_inputs(const fix_attn_desc *d, const void *q, const void *k, void *ws, size_t ws_bytes,
                                 void *hip_stream) {
  const fix_status v = fix_attn_validate(d);
  if (v != FIX_OK) return v;
  if (!q || !k || !ws) return FIX_E_INVALID;
  if (ws_bytes < 8) return FIX_E_WORKSPACE;
  const hipStream_t st = (hipStream_t)hip_stream;
  const bool f32in = d->in_dtype == FIX_F32;
  const int64_t nt = d->cu_seqlens ? d->T : d->B * d->T;
  unsigned *mx = (unsigned *)ws;
  hipError_t e = hipMemsetAsync(mx, 0, 8, st);
  if (e == hipSuccess) e = fix::launch_absmax(q, f32in, nt * d->Hq * d->dk, mx, st);
  if (e == hipSuccess) e = fix::launch_absmax(k, f32in, nt * d->Hkv * d->dk, mx + 1, st);
  unsigned h[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(h, mx, 8, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  const unsigned lim = 0x477FE000u;  // 65504.0f, the largest finite fp16
  return (h[0] > lim || h[1] > lim) ? FIX_E_RANGE : FIX_OK;
}

const char *fix_attn_status_string(fix_status s) {
  switch (s) {
    case FIX_OK: return "ok";
    case FIX_E_INVALID: return "invalid argument";
    case FIX_E_UNSUPPORTED: return "unsupported shape or head dimension (head dims must be 16, 32, 64 or 128)";
    case FIX_E_WORKSPACE: return "workspace too small";
    case FIX_E_HIP: return "HIP launch failed";
    case FIX_E_RANGE: return "q or k holds a value the fp16 operands cannot hold (|x| > 65504, inf or NaN)";
  }
  return "unknown status";
}

int fix_attn_last_hip_error(void) { return g_last_hip_error; }

void fix_attn_set_event_trace(void **events, int capacity) {
  g_trace.events = (hipEvent_t *)events;
  g_trace.capacity = events ? capacity : 0;
  g_trace.count = 0;
}

int fix_attn_event_trace_count(void) { return g_trace.count; }

const char *fix_attn_event_trace_label(int i) {
  if (i < 1 || i >= g_trace.count) return nullptr;
  return g_trace.labels[i];
}

}  // extern "C"
