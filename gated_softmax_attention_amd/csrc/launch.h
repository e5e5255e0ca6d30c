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

// Scalar-gate (forgetting-attention) forward, fox.hip.
struct FoxArgs {
  const void *q, *k;
  const _Float16 *V16;  // [T, Hkv, DV] v as fp16
  const float *loc;     // [T, Hkv] log2 gate prefix local to the token's 64-token block
  const double *ref;    // [64-block][Hkv] log2 gate prefix before each block
  const void *w, *z;
  void *o;
  float *m, *rstd, *x;
  Plan plan;
  int Hq, Hkv;
  float sl2, eps;
  int o_norm, out_f32;
};
hipError_t launch_fox_prefix(const float *g, bool logits, const Plan &plan, int nseq, int Hkv, float *loc,
                             double *ref, hipStream_t st);
hipError_t launch_fox_fwd(int dk, int dv, bool f32in, const FoxArgs &a, int grid, hipStream_t st);

// Scalar-gate backward (fox_bwd.h): the logit-bias form of the gradients.
// Operands are fp16 copies, rows padded to 32 columns where a product reads
// them column-wise (head dims below 32).
struct FoxBwdArgs {
  const _Float16 *Q16;  // [T, Hq, DKP]
  const _Float16 *K16;  // [T, Hkv, DKP]
  const _Float16 *V16;  // [T, Hkv, DV]
  const _Float16 *D16;  // [T, Hq, DVP] sigma * delta (delta: the gradient reaching x)
  const float *mb;      // [T, Hq] m log2e - e (sigma = 2^-e)
  const float *loc;     // [T, Hkv] log2 gate prefix local to the token's 64-token block
  const double *ref;    // [64-block][Hkv] log2 gate prefix before each block
  float *rsum;          // [T, Hq] row sums of dS (written by the dq kernel)
  float *csum;          // [T, Hkv] column sums of dS over the head group (dk/dv kernel)
  void *dq, *dk, *dv;
  Plan plan;
  int Hq, Hkv;
  float sl2, scale;
  int out_f32;
};
struct FoxPrepArgs {
  const float *x, *rstd, *m;
  const void *dO, *z, *w;
  Plan plan;
  int Hq, Hkv;
  int o_norm, out_f32, in_f32;
  _Float16 *D16;   // [T, Hq, DVP]
  float *mb;       // [T, Hq]
  void *dz;        // [T, Hq, DV] or null
  float *dw_part;  // [128-chunks * Hkv][DV] or null
};
enum FoxBwdKernel { FK_DQ = 0, FK_DKV = 1 };
hipError_t launch_fox_bwd_prep(int dv, const FoxPrepArgs &a, int ncb_ub, hipStream_t st);
hipError_t launch_fox_bwd_d16(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fox_bwd_d32(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fox_bwd_d64(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st);
hipError_t launch_fox_bwd_d128(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st);
inline hipError_t launch_fox_bwd(FoxBwdKernel kind, int dk, int dv, const FoxBwdArgs &a, int grid, hipStream_t st) {
  switch (dk) {
    case 16: return launch_fox_bwd_d16(kind, dv, a, grid, st);
    case 32: return launch_fox_bwd_d32(kind, dv, a, grid, st);
    case 64: return launch_fox_bwd_d64(kind, dv, a, grid, st);
    case 128: return launch_fox_bwd_d128(kind, dv, a, grid, st);
  }
  return hipErrorInvalidValue;
}
// dg_t = sum over t' >= t of the sequence of (sum over the group of rsum - csum)
// (times sigmoid(-x) when the gate was given as logits x).
hipError_t launch_fox_dg_scan(const float *rsum, const float *csum, const float *logits, const Plan &plan, int nseq,
                              int Hq, int Hkv, float *dg, hipStream_t st);
// fp16 copy of a [rows, D] bf16 or fp32 tensor into [rows, DP] (DP >= D, zero columns past D).
hipError_t launch_to_f16_pad(const void *in, bool in_f32, int64_t rows, int D, int DP, _Float16 *out, hipStream_t st);

struct BwdArgs {
  const void *q, *k, *v;
  const float *Gl2, *Gam;      // 128-chunk local prefix sums of g (log2 units), chunk decays
  const double *Lam;           // [chunk][Hkv][DV] prefix over chunks of the chunk log2 totals
  const _Float16 *Vr;          // [chunk][Hkv][CB][DV] V scaled to its chunk end
  const _Float16 *Kt;          // [chunk][Hkv][DK][CB] transposed fp16 K tiles (key_pos order)
  const _Float16 *Q16;         // [T, Hq, DK] q as fp16 (exact for |q| in [2^-14, 65504])
  // what the gradient reaching x (delta) is recomputed from, element by
  // element, where the exact-decay paths need it (the preprocess keeps only
  // its scaled fp16 forms): x, rstd, the row projection prj, dO, z, w
  const float *x, *rstd, *prj;
  const void *dO, *z, *w;
  int o_norm;
  const _Float16 *dh;          // [T, Hq, DV] sigma * exp(Gl) * delta
  const _Float16 *dhT;         // [chunk][Hq][DV][CB] the same as transposed tiles (key_pos order)
  const float *mb, *sig;       // [T, Hq] m log2e - e, sigma = 2^-e
  const float *qside;          // [T, Hkv, DV]
  // Operands of the pairs in the same or the adjacent chunk, relative to
  // 32-token blocks (blocks tile every 128-chunk):
  const _Float16 *VE;          // [T, Hkv, DV] exp(Gl_blockend - Gl_j) v_j
  const __bf16 *VBH, *VBL;     // [T, Hkv, DV] exp(Gl_blockstart-1 - Gl_j) v_j (>= |v_j|), bf16 hi / lo
  const _Float16 *X16;         // [T, Hq, DV] exp(Gl_i - Gl_blockstart-1) sigma delta_i
  const __bf16 *XH, *XL;       // the same, bf16 hi and lo parts
  float *dq_i, *dk_i, *dv_i;   // within-chunk contributions (fp32)
  void *dq, *dk, *dv;          // outputs (out dtype)
  float *dG;                   // [T, Hkv, DV] gradient with respect to the prefix sums of g
  float *dg_tot;               // [chunk][Hkv][4][DV] dG summed over each 32-key block of the chunk
  Plan plan;
  int Hq, Hkv;
  float sl2, scale;
  int out_f32;
};

struct PrepArgs {
  const float *x, *rstd, *m, *Gl2;
  const void *dO, *z, *w;
  Plan plan;
  int Hq, Hkv;
  int o_norm, out_f32, in_f32;
  float *prj;          // [Ttot, Hq] the row projection of the norm's backward (o_norm only)
  _Float16 *dh;        // [Ttot, Hq, DV] fp16, sigma * exp(Gl) * delta
  float *mb;           // [Ttot, Hq] m log2e - e
  float *sig;          // [Ttot, Hq] sigma = 2^-e
  float *qside;        // [Ttot, Hkv, DV] sum over the group of delta (.) x
  void *dz;            // [Ttot, Hq, DV] out dtype, or null
  float *dw_part;      // [chunks * Hkv][DV] per-block partial sums of dn (.) xh, or null
  _Float16 *X16;       // [Ttot, Hq, DV] sigma * exp(Gl - Gl at the token before the 32-block) * delta
  __bf16 *XH, *XL;     // the same as bf16 hi / lo parts
};

hipError_t launch_plan(const int64_t *cu, int nseq, int T, int64_t Ttot, const Plan &plan, hipStream_t st);
hipError_t launch_gate_prep(int dv, const float *g, bool logits, const void *v, bool in_f32, const Plan &plan,
                            int Hkv, int nch_ub, float *Gl2, float *Gam, _Float16 *VtT, hipStream_t st);
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

hipError_t launch_gate_prep_rows(int dv, const float *g, bool logits, const void *v, bool in_f32, const Plan &plan,
                                 int Hkv, int ncb_ub, float *Gl2, float *Gam, _Float16 *Vr, _Float16 *VE, __bf16 *VBH,
                                 __bf16 *VBL, hipStream_t st);
hipError_t launch_chunk_logprefix(int dv, const float *Gl2, const Plan &plan, int Hkv, double *Lam, hipStream_t st);
// Decode cache (layout in decode.hip): device pointers carved from one
// caller buffer, and the shape they were carved for.
struct DecodeCache {
  int B, cap, Hq, Hkv, G, dk, dv;
  int *len;
  _Float16 *K, *VT, *Vo;
  float *Go;
  double *Lam;
};
hipError_t launch_decode_reset(const DecodeCache &dc, hipStream_t st);
hipError_t launch_decode_append(const DecodeCache &dc, const void *k, const void *v, const float *g, int n,
                                const int *n_seq, bool in_f32, bool logits, hipStream_t st);
hipError_t launch_decode_open(const DecodeCache &dc, _Float16 *vto, hipStream_t st);
hipError_t launch_decode_step(const DecodeCache &dc, const void *q, bool in_f32, float sl2, int splits,
                              const _Float16 *vto, float *part, float *mpart, hipStream_t st);
hipError_t launch_decode_combine(const DecodeCache &dc, int units, const float *part, const float *mpart,
                                 const void *w, const void *z, bool in_f32, bool out_f32, bool o_norm, float eps,
                                 void *o, float *m, hipStream_t st);
hipError_t launch_to_f16(const void *in, bool in_f32, int64_t n, _Float16 *out, hipStream_t st);
hipError_t launch_absmax(const void *in, bool in_f32, int64_t n, unsigned *out, hipStream_t st);
hipError_t launch_tiles_t(int D, const void *in, int in_kind, const Plan &plan, int H, int ncb_ub, _Float16 *out,
                          hipStream_t st);
hipError_t launch_bwd_prep(int dv, const PrepArgs &a, int ncb_ub, hipStream_t st);
hipError_t launch_dw_reduce(const float *part, const int *counts, int Hkv, int dv, float *dw, hipStream_t st);
// logits != null: the gate was given as logits x; dg is multiplied by dg/dx = sigmoid(-x).
hipError_t launch_dg_scan(int dv, const float *dG, const float *logits, const Plan &plan, int Hkv, int ncb_ub,
                          float *tot, float *carry, float *dg, hipStream_t st);

// Backward MFMA kernels, one translation unit per dk.
enum BwdKernel { BK_INTRA_DQ = 0, BK_INTRA_DKV = 1, BK_DQ = 2, BK_DKV = 3 };
hipError_t launch_bwd_d16(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st);
hipError_t launch_bwd_d32(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st);
hipError_t launch_bwd_d64(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st);
hipError_t launch_bwd_d128(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st);

inline hipError_t launch_bwd(BwdKernel kind, int dk, int dv, bool f32in, const BwdArgs &a, dim3 grid,
                             hipStream_t st) {
  switch (dk) {
    case 16: return launch_bwd_d16(kind, dv, f32in, a, grid, st);
    case 32: return launch_bwd_d32(kind, dv, f32in, a, grid, st);
    case 64: return launch_bwd_d64(kind, dv, f32in, a, grid, st);
    case 128: return launch_bwd_d128(kind, dv, f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fix
